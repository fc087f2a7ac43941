"""GPU parity: every stage of the HIP path, called through the C ABI, against
the float64 oracle on the same seeded inputs.  Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from post_weight_quantization_syrk_amd import gptq, synth
from gpu_util import DEV, dev_bf16, dev_f32, spd_u_bar
from gpu_util import gpu_quant as _gpu_quant
from parity import check_row_losses, compare_quant, h_rel_error

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    gptq.lib()  # loud failure if the library is missing


def to_dev(a, dtype):
    return dev_bf16(a) if dtype == "bf16" else dev_f32(a)


def rand_x(n, d, dtype, seed, ld=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, ld or d), dtype=np.float32) * np.exp(
        rng.standard_normal(ld or d)).astype(np.float32)
    if dtype == "bf16":
        b = synth.f32_to_bf16_bits(x)
        return b, synth.as_f64(b, "bf16")[:, :d]
    return x, x.astype(np.float64)[:, :d]


# ------------------------------------------------------------------ Hessian
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,d", [(1, 1), (100, 37), (1000, 300), (3000, 513), (640, 256)])
def test_hessian_small_ragged(dtype, n, d):
    print(f"[hessian] dtype={dtype} n={n} d={d}", flush=True)
    xs, x64 = rand_x(n, d, dtype, seed=n * 7 + d)
    X = to_dev(xs, dtype)
    H = torch.zeros((d, d), dtype=torch.float32, device=DEV)
    sentinel = 12345.0
    H += torch.triu(torch.full((d, d), sentinel, device=DEV), 1)
    gptq.gptq_hessian_accumulate(H, X)
    Hn = H.cpu().numpy()
    ref = oracle.hessian([x64])
    assert h_rel_error(Hn, ref) <= 1e-5 if dtype == "f32" else h_rel_error(Hn, ref) <= 1e-5
    assert np.all(np.triu(Hn, 1) == np.triu(np.full((d, d), sentinel, np.float32), 1))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hessian_strided_rows_and_accumulation(dtype):
    n, d, ld = 2000, 200, 203     # odd row stride: unaligned rows, scalar load path
    xs, x64 = rand_x(n, d, dtype, seed=5, ld=ld)
    X = to_dev(xs, dtype)
    H = torch.zeros((d, d), dtype=torch.float32, device=DEV)
    gptq.gptq_hessian_accumulate(H, X[:700])
    gptq.gptq_hessian_accumulate(H, X[700:])
    assert h_rel_error(H.cpu().numpy(), oracle.hessian([x64])) <= 1e-5


def test_hessian_deterministic():
    xs, _ = rand_x(5000, 640, "bf16", seed=9)
    X = dev_bf16(xs)
    outs = []
    for _ in range(2):
        H = torch.zeros((640, 640), dtype=torch.float32, device=DEV)
        gptq.gptq_hessian_accumulate(H, X)
        outs.append(H.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_hessian_small_workload():
    wl = synth.SMALL
    xs = synth.x_chunk(wl, 0)
    H = torch.zeros((wl.d_in, wl.d_in), dtype=torch.float32, device=DEV)
    gptq.gptq_hessian_accumulate(H, dev_f32(xs))
    ref = oracle.hessian([synth.as_f64(xs, "f32")])
    assert h_rel_error(H.cpu().numpy(), ref) <= 1e-6


# ------------------------------------------------------------ factorization
def _spd(d, seed, n=None):
    rng = np.random.default_rng(seed)
    n = n or 3 * d
    x = rng.standard_normal((n, d)) @ (np.eye(d) + 0.3 * rng.standard_normal((d, d)) / np.sqrt(d))
    x *= np.exp(0.5 * rng.standard_normal(d))
    return (2.0 * x.T @ x).astype(np.float32)


@pytest.mark.parametrize("d", [1, 5, 64, 100, 130, 256, 1000, 2150, 3000, 4096, 5000])
def test_prepare_matches_oracle(d):
    H32 = _spd(d, d)
    H = dev_f32(np.tril(H32))
    U, dead, status = gptq.gptq_prepare_hinv(H, damp=0.01)
    ref = oracle.prepare(H32.astype(np.float64), 0.01)
    Ug = U.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(Ug - ref["U"])) / np.max(np.abs(ref["U"]))
    # fp32 bar: U's entries come out of O(d)-long chains of rounded fp32
    # products (factorization, then triangular inverse); with independent
    # rounding errors the relative error grows like sqrt(d) u (u = 2^-24)
    bar = spd_u_bar(d)
    print(f"[prepare] d={d} max rel U err {err:.2e} (bar {bar:.2e})", flush=True)
    assert err <= bar
    assert np.all(np.tril(Ug, -1) == 0)
    np.testing.assert_allclose(H.cpu().numpy(), ref["H"], rtol=2e-7, atol=0)
    assert not dead.cpu().numpy().any()


def test_prepare_dead_channels_and_identity():
    d = 130
    H32 = _spd(d, 3)
    H32[:, [4, 77]] = 0
    H32[[4, 77], :] = 0
    H = dev_f32(H32)
    U, dead, _ = gptq.gptq_prepare_hinv(H)
    ref = oracle.prepare(H32.astype(np.float64))
    assert dead.cpu().numpy().astype(bool).tolist() == ref["dead"].tolist()
    err = np.max(np.abs(U.cpu().numpy() - ref["U"])) / np.max(np.abs(ref["U"]))
    assert err <= spd_u_bar(d)
    # H = 2I: U is exactly diagonal
    U, _, _ = gptq.gptq_prepare_hinv(dev_f32(2 * np.eye(256)))
    Un = U.cpu().numpy()
    assert np.count_nonzero(Un - np.diag(np.diag(Un))) == 0


def test_prepare_not_spd():
    d = 70
    with pytest.raises(gptq.NotSPDError) as e:
        gptq.gptq_prepare_hinv(dev_f32(-np.eye(d)))
    assert e.value.pivot == d  # elimination starts at index d-1
    with pytest.raises(oracle.NotSPD):
        oracle.prepare(-np.eye(d))
    # indefinite with a positive diagonal
    A = np.eye(4, dtype=np.float32)
    A[3, 2] = A[2, 3] = 2.0
    with pytest.raises(gptq.NotSPDError):
        gptq.gptq_prepare_hinv(dev_f32(A), damp=0.0)
    with pytest.raises(oracle.NotSPD):
        oracle.prepare(A.astype(np.float64), damp=0.0)


# ---------------------------------------------------------------- quantizer
QCASES = [(4, 128, False), (4, 64, True), (3, 64, True), (3, 32, False), (2, 32, False),
          (4, -1, False), (2, -1, True)]


@pytest.mark.parametrize("bits,g,sym", QCASES)
@pytest.mark.parametrize("d_out,d_in", [(37, 256), (16, 128), (5, 320), (64, 384)])
def test_identity_hessian_bit_exact_rtn(bits, g, sym, d_out, d_in):
    if g > 0 and d_in % g:
        pytest.skip("group must divide d_in")
    print(f"[rtn] bits={bits} g={g} sym={sym} {d_out}x{d_in}", flush=True)
    rng = np.random.default_rng(bits * 1000 + d_in + d_out)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    W[d_out // 2, d_in // 3] = 0.7
    W[0, :32] = 0.0  # a degenerate group
    U, dead, _ = gptq.gptq_prepare_hinv(dev_f32(2 * np.eye(d_in)))
    out = _gpu_quant(dev_f32(W), U, dead, bits, g, sym)
    ref = oracle.rtn(W.astype(np.float64), bits=bits, group_size=g, sym=sym)
    np.testing.assert_array_equal(out["scales"], ref["scales"])
    np.testing.assert_array_equal(out["zeros"], ref["zeros"])
    np.testing.assert_array_equal(out["codes"], ref["codes"])


def _tie_rows(bits, sym, d_in, g, seed):
    """Rows whose groups have exact binary16 steps and values placed exactly on
    half steps (ties) and one float32 ulp either side of them."""
    rng = np.random.default_rng(seed)
    maxq = (1 << bits) - 1
    steps = [2.0 ** -4, 3.0 / 64, 5.0 / 128, 2.0 ** -7, 7.0 / 256]
    rows = []
    for r in range(len(steps) * 2):
        s = steps[r % len(steps)]
        row = np.zeros(d_in, np.float32)
        for g0 in range(0, d_in, g):
            if sym:
                amax = maxq * s / 2.0          # fp16(2 amax / maxq) = s exactly
                lo_k, hi_k = -(maxq + 1) // 2, (maxq - 1) // 2
                v = [amax]
            else:
                z0 = int(rng.integers(0, maxq + 1))
                lo_k, hi_k = -z0, maxq - z0
                v = [lo_k * s, hi_k * s]        # range [lo, hi]: step (hi - lo)/maxq = s
            while len(v) < g:
                k = int(rng.integers(lo_k, hi_k))
                t = np.float32((k + 0.5) * s)
                kind = int(rng.integers(0, 3))
                if kind == 1:
                    t = np.nextafter(t, np.float32(np.inf))
                elif kind == 2:
                    t = np.nextafter(t, np.float32(-np.inf))
                v.append(float(t))
            row[g0:g0 + g] = rng.permutation(np.array(v[:g], np.float32))
        rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("bits,sym", [(4, False), (4, True), (3, False), (2, True)])
def test_rtn_exact_ties(bits, sym):
    """Quotients exactly at k + 1/2 round to the even code; one ulp away they
    round to the nearer one (identity Hessian: the result is plain rounding)."""
    d_in, g = 128, 32
    W = _tie_rows(bits, sym, d_in, g, seed=bits * 10 + int(sym))
    print(f"[ties] bits={bits} sym={sym} {W.shape}", flush=True)
    U, dead, _ = gptq.gptq_prepare_hinv(dev_f32(2 * np.eye(d_in)))
    out = _gpu_quant(dev_f32(W), U, dead, bits, g, sym)
    ref = oracle.rtn(W.astype(np.float64), bits=bits, group_size=g, sym=sym)
    np.testing.assert_array_equal(out["scales"], ref["scales"])
    np.testing.assert_array_equal(out["zeros"], ref["zeros"])
    np.testing.assert_array_equal(out["codes"], ref["codes"])


@pytest.mark.parametrize("bits,g,sym", QCASES)
def test_quantize_parity_correlated(bits, g, sym):
    d_out, d_in = 96, 384
    H32 = _spd(d_in, 11)
    rng = np.random.default_rng(12)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    U, dead, _ = gptq.gptq_prepare_hinv(dev_f32(H32))
    out = _gpu_quant(dev_f32(W), U, dead, bits, g, sym)
    p = oracle.prepare(H32.astype(np.float64))
    ref = oracle.gptq(W, p["U"], p["dead"], bits=bits, group_size=g, sym=sym, block=128)
    rep = compare_quant(out, ref, group_size=g, bits=bits, W=W.astype(np.float64),
                        H0=H32.astype(np.float64))
    print(f"[quant] bits={bits} g={g} sym={sym} {rep}", flush=True)
    # the damped-H loss identity holds on the GPU side too (rows on the same
    # greedy path to fp32 rounding; the layer total within 1e-3)
    check_row_losses(out["loss"], out, ref)


@pytest.mark.parametrize("d_in,wdt", [(256, "f32"), (256, "bf16"), (100, "f32"), (100, "bf16")])
def test_quantize_dead_columns(d_in, wdt):
    """Channels with H_ii = 0 (inputs that never fire): prepare flags them and
    the quantizer zeroes those columns of W before the loop ([P1] 阶段一's
    dead-column handling), on the 8-wide and the scalar conversion paths."""
    d_out = 48
    H32 = _spd(d_in, 21)
    dead_idx = np.array([0, 7, d_in // 2, d_in - 1])
    H32[dead_idx, :] = 0.0
    H32[:, dead_idx] = 0.0
    rng = np.random.default_rng(22)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    if wdt == "bf16":
        Wb = synth.f32_to_bf16_bits(W)
        W_dev, W64 = dev_bf16(Wb), synth.as_f64(Wb, "bf16")
    else:
        W_dev, W64 = dev_f32(W), W.astype(np.float64)
    print(f"[dead] d_in={d_in} {wdt}", flush=True)
    U, dead, status = gptq.gptq_prepare_hinv(dev_f32(np.tril(H32)))
    out = _gpu_quant(W_dev, U, dead, 4, -1, False)
    p = oracle.prepare(H32.astype(np.float64))
    assert dead.cpu().numpy().astype(bool).tolist() == p["dead"].tolist()
    ref = oracle.gptq(W64, p["U"], p["dead"], bits=4, group_size=-1, sym=False, block=128)
    rep = compare_quant(out, ref, group_size=-1, bits=4, W=W64, H0=H32.astype(np.float64))
    print(f"[dead] {rep}", flush=True)
    # a dead column quantizes the zero it was set to
    deq = out["scales"][:, :1] * (out["codes"][:, dead_idx].astype(np.float64) - out["zeros"][:, :1])
    np.testing.assert_array_equal(deq, 0.0)


def test_quantize_empty_rows():
    U, dead, _ = gptq.gptq_prepare_hinv(dev_f32(2 * np.eye(128)))
    W = torch.zeros((0, 128), dtype=torch.float32, device=DEV)
    codes, scales, zeros, _ = gptq.gptq_quantize_layer(W, U, dead)
    assert codes.shape == (0, 128)


# --------------------------------------------------------------------- pack
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d_in,g,sym", [(32, 32, False), (100, -1, True), (4096, 128, False),
                                        (320, 64, True)])
def test_pack_bit_exact(bits, d_in, g, sym):
    rng = np.random.default_rng(bits + d_in)
    d_out = 7
    codes = rng.integers(0, 1 << bits, size=(d_out, d_in), dtype=np.uint8)
    ng = 1 if g == -1 else d_in // g
    scales = oracle.fp16_rne(np.exp(rng.standard_normal((d_out, ng)) - 5))
    zeros = rng.integers(0, 1 << bits, size=(d_out, ng)).astype(np.float64)
    cd = torch.from_numpy(codes).to(DEV)
    qw, s16, z16 = gptq.gptq_pack(cd, dev_f32(scales), dev_f32(zeros), bits=bits, group_size=g,
                                  sym=sym)
    torch.cuda.synchronize()
    ref = oracle.pack_rows(codes, bits)
    np.testing.assert_array_equal(qw.cpu().numpy().view(np.uint32), ref)
    np.testing.assert_array_equal(s16.cpu().numpy().view(np.uint16), oracle.fp16_bits(scales))
    if not sym:
        np.testing.assert_array_equal(z16.cpu().numpy().view(np.uint16), oracle.fp16_bits(zeros))


# -------------------------------------------------------------- end to end
def _e2e(wl: synth.Workload, tensor=0):
    """All four calls through the C ABI vs the oracle on the same inputs."""
    print(f"[e2e] {wl.name}", flush=True)
    Wst = synth.w_matrix(wl, tensor)
    W64 = synth.as_f64(Wst, wl.w_dtype)
    chunks = [synth.x_chunk(wl, c) for c in range(synth.n_chunks(wl))]
    H = torch.zeros((wl.d_in, wl.d_in), dtype=torch.float32, device=DEV)
    for xc in chunks:
        gptq.gptq_hessian_accumulate(H, to_dev(xc, wl.x_dtype))
    H_gpu = H.cpu().numpy()
    U, dead, _ = gptq.gptq_prepare_hinv(H, damp=wl.damp)
    out = _gpu_quant(to_dev(Wst, wl.w_dtype), U, dead, wl.bits, wl.group_size, wl.sym)
    H0 = oracle.hessian(synth.as_f64(xc, wl.x_dtype) for xc in chunks)
    assert h_rel_error(H_gpu, H0) <= 1e-4
    p = oracle.prepare(H0, wl.damp)
    ref = oracle.gptq(W64, p["U"], p["dead"], bits=wl.bits, group_size=wl.group_size,
                      sym=wl.sym, block=wl.block)
    rep = compare_quant(out, ref, group_size=wl.group_size, bits=wl.bits, W=W64, H0=H0)
    print(f"[e2e] {wl.name}: {rep}", flush=True)
    return rep


def test_e2e_small_workload():
    _e2e(synth.SMALL)


@pytest.mark.parametrize("wl", [
    synth.scaled(synth.ATTN7B, d_out=512, d_in=1024, n_tokens=16384, chunk_tokens=4096),
    synth.scaled(synth.FFN_GATE, d_out=700, d_in=512, n_tokens=8192, chunk_tokens=4096),
    synth.scaled(synth.FFN_DOWN, d_out=256, d_in=1408, n_tokens=8192, chunk_tokens=4096),
    synth.scaled(synth.L70B_SQ, d_out=300, d_in=1024, n_tokens=8192, bits=2, group_size=32),
    synth.scaled(synth.L70B_SQ, d_out=300, d_in=1024, n_tokens=8192, bits=4, group_size=-1),
    # d_in not a multiple of 4: the trailing updates stage their operands
    # element by element (650 = 5 x 128 + 10, ragged last block)
    synth.scaled(synth.L70B_SQ, d_out=200, d_in=650, n_tokens=4096, bits=4, group_size=-1),
    # 1028 = 8 x 128 + 4: vector staging with a 4-column last tile
    synth.scaled(synth.L70B_SQ, d_out=136, d_in=1028, n_tokens=4096, bits=3, group_size=-1),
], ids=lambda w: w.name)
def test_e2e_scaled_workloads(wl):
    _e2e(wl)


def test_quantize_full_size_attention_layer():
    """4096 x 4096 bf16 layer at full size, stage-isolated from the Hessian:
    the oracle's own H from 16384 seeded tokens feeds both sides."""
    wl = synth.ATTN7B
    sub = synth.scaled(wl, n_tokens=16384, chunk_tokens=8192)
    H0 = oracle.hessian(synth.as_f64(synth.x_chunk(sub, c), "bf16") for c in range(2))
    H32 = np.tril(H0).astype(np.float32)
    H0r = np.tril(H32).astype(np.float64)
    H0r = H0r + np.tril(H0r, -1).T
    Wst = synth.w_matrix(wl)
    W64 = synth.as_f64(Wst, "bf16")
    U, dead, _ = gptq.gptq_prepare_hinv(dev_f32(H32), damp=wl.damp)
    out = _gpu_quant(dev_bf16(Wst), U, dead, wl.bits, wl.group_size, wl.sym)
    print("[quant full] oracle running", flush=True)
    p = oracle.prepare(H0r, wl.damp)
    ref = oracle.gptq(W64, p["U"], p["dead"], bits=wl.bits, group_size=wl.group_size,
                      sym=wl.sym, block=128)
    rep = compare_quant(out, ref, group_size=wl.group_size, bits=wl.bits, W=W64, H0=H0r)
    print(f"[quant full] {rep}", flush=True)


def test_trailing_staging_paths_agree():
    """The trailing update loads its operands as 16-byte vectors when d_in is
    a multiple of 4 and U is 16-byte aligned, and element by element
    otherwise.  Both feed the same three bf16 parts to the same products in
    the same order, so the results agree bit for bit; a copy of U at a 4-byte
    offset takes the element-wise path on the same layer."""
    d_out, d_in = 200, 640
    rng = np.random.default_rng(640)
    A = rng.standard_normal((d_in + 96, d_in)) * np.exp(0.5 * rng.standard_normal(d_in))
    H = (2.0 / A.shape[0]) * (A.T @ A)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    U, dead, _ = gptq.gptq_prepare_hinv(dev_f32(H))
    buf = torch.empty(d_in * d_in + 1, dtype=torch.float32, device=DEV)
    U_off = buf[1:].view(d_in, d_in)
    U_off.copy_(U)
    assert U.data_ptr() % 16 == 0 and U_off.data_ptr() % 16 != 0
    print(f"[staging] {d_out}x{d_in}: aligned U against U at a 4-byte offset", flush=True)
    for bits, g, sym in [(4, 128, False), (3, -1, True)]:
        a = _gpu_quant(dev_f32(W), U, dead, bits, g, sym)
        b = _gpu_quant(dev_f32(W), U_off, dead, bits, g, sym)
        for key in ("codes", "scales", "zeros", "loss"):
            np.testing.assert_array_equal(a[key], b[key])


def test_side_stream_calls_match_current_stream():
    """Every call launched on a stream other than the current one, with its
    scratch allocated by the binding (on that stream), gives the same bits as
    on the current stream; the side stream's work is not disturbed by
    allocations made meanwhile on the current one."""
    wl = synth.scaled(synth.ATTN7B, d_out=320, d_in=384, n_tokens=3000, chunk_tokens=3000)
    xb = dev_bf16(synth.x_chunk(wl, 0))
    W = dev_bf16(synth.w_matrix(wl))

    def run(stream):
        H = torch.zeros((wl.d_in, wl.d_in), dtype=torch.float32, device=DEV)
        gptq.gptq_hessian_accumulate(H, xb, stream=stream)
        U, dead, st = gptq.gptq_prepare_hinv(H, wl.damp, stream=stream)
        out = gptq.gptq_quantize_layer(W, U, dead, bits=4, group_size=128, stream=stream)
        # churn on the current stream while the side stream may still run
        for _ in range(4):
            torch.empty(8 << 20, dtype=torch.uint8, device=DEV).fill_(0xAB)
        (torch.cuda.current_stream() if stream is None else stream).synchronize()
        return [t.cpu() for t in (H, U) + tuple(out[:3])]

    ref = run(None)
    side = torch.cuda.Stream()
    got = run(side)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_far_update_tile_shapes_agree_and_match_oracle():
    """A layer tall enough for the 128 x 128 far-update tiles (65536 rows x 1024:
    2048 of them) against the same first 4096 rows quantized alone (128 x 64
    tiles): every element sums the same part products in the same k order, so
    the two must agree bit for bit; and 32 sampled rows against the oracle."""
    d_out, d_in = 65536, 1024
    H32 = _spd(d_in, 21)
    rng = np.random.default_rng(22)
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    U, dead, _ = gptq.gptq_prepare_hinv(dev_f32(H32))
    print("[far tiles] 65536 rows", flush=True)
    tall = _gpu_quant(dev_f32(W), U, dead, 4, 128, False)
    print("[far tiles] 4096 rows", flush=True)
    part = _gpu_quant(dev_f32(W[:4096]), U, dead, 4, 128, False)
    for k in ("codes", "scales", "zeros", "loss"):
        np.testing.assert_array_equal(tall[k][:4096], part[k])
    rows = np.sort(np.random.default_rng(23).choice(d_out, 32, replace=False))
    p = oracle.prepare(H32.astype(np.float64))
    ref = oracle.gptq(W[rows].astype(np.float64), p["U"], p["dead"], bits=4, group_size=128,
                      sym=False, block=128)
    sub = {k: v[rows] for k, v in tall.items()}
    rep = compare_quant(sub, ref, group_size=128, bits=4, W=W[rows].astype(np.float64),
                        H0=H32.astype(np.float64))
    print(f"[far tiles] {rep}", flush=True)
