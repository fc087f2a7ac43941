"""GPU parity of the dequantized 4-bit product (gptq_w4a16_matmul) against the
float64 oracle ([P1] 阶段三; [P5] 存储代价).

Bar: every product x (q - z) is exact in fp32 and only the sums round, so
|Y_gpu - Y_ref| <= (K + 2) u sum_k |x_k| |W_hat_nk| (u = 2^-24), the
worst-case bound of fp32 accumulation of K terms plus the scaling and the
cross-group additions.  The packed inputs are made with the oracle's
packing, never with the GPU path."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from post_weight_quantization_syrk_amd import gptq, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U32 = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    gptq.lib()


def make(m, d_in, d_out, g, sym, seed, ld=None):
    rng = np.random.default_rng(seed)
    G = d_in if g == -1 else g
    ng = d_in // G
    codes = rng.integers(0, 16, size=(d_out, d_in), dtype=np.uint8)
    scales = oracle.fp16_rne(np.exp(rng.uniform(-6.0, -2.0, size=(d_out, ng))))
    zeros = rng.integers(0, 16, size=(d_out, ng)).astype(np.float64)
    qw = oracle.pack_rows(codes, 4)
    s16 = oracle.fp16_bits(scales)
    z16 = oracle.fp16_bits(zeros)
    x = rng.standard_normal((m, ld or d_in), dtype=np.float32)
    xb = synth.f32_to_bf16_bits(x)
    return xb, synth.as_f64(xb, "bf16")[:, :d_in], qw, s16, z16


def run(xb, qw, s16, z16, d_in, g, sym):
    X = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)[:, :d_in]
    Q = torch.from_numpy(qw.astype(np.uint32).view(np.int32)).to(DEV)
    S = torch.from_numpy(s16.view(np.int16)).to(DEV)
    Z = torch.from_numpy(z16.view(np.int16)).to(DEV)
    Y = gptq.gptq_w4a16_matmul(X, Q, S, None if sym else Z, group_size=g, sym=sym)
    torch.cuda.synchronize()
    return Y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,d_in,d_out,g,sym,ld", [
    (1, 128, 8, 128, False, None),
    (37, 256, 100, 64, False, None),
    (128, 384, 256, 32, True, None),
    (300, 1024, 520, 128, False, 1032),
    (200, 512, 130, -1, False, None),
    (64, 4096, 4096, 128, False, None),
])
def test_w4a16_matches_oracle(m, d_in, d_out, g, sym, ld):
    print(f"[w4a16] m={m} d_in={d_in} d_out={d_out} g={g} sym={sym} ld={ld}", flush=True)
    xb, x64, qw, s16, z16 = make(m, d_in, d_out, g, sym, seed=m + d_in + d_out, ld=ld)
    Y = run(xb, qw, s16, z16, d_in, g, sym)
    ref = oracle.dequant_matmul(x64, qw, s16, None if sym else z16, bits=4, group_size=g,
                                sym=sym)
    What = oracle.dequantize(qw, s16, None if sym else z16, bits=4, group_size=g, sym=sym,
                             d_in=d_in)
    bound = (d_in + 2) * U32 * (np.abs(x64) @ np.abs(What).T)
    err = np.abs(Y - ref)
    print(f"[w4a16] max err / bound {float((err / np.maximum(bound, 1e-300)).max()):.3e}, "
          f"max rel {float((err / np.maximum(np.abs(ref), 1e-30)).max()):.3e}", flush=True)
    assert np.all(err <= bound)


def test_w4a16_identity_rows_give_w_hat():
    # X = rows of the identity: Y is W_hat transposed, exactly (one product per sum)
    d_in, d_out = 256, 64
    xb, _, qw, s16, z16 = make(8, d_in, d_out, 64, False, seed=5)
    eye = np.zeros((d_in, d_in), dtype=np.float32)
    eye[np.arange(d_in), np.arange(d_in)] = 1.0
    xb = synth.f32_to_bf16_bits(eye)
    Y = run(xb, qw, s16, z16, d_in, 64, False)
    What = oracle.dequantize(qw, s16, z16, bits=4, group_size=64, sym=False, d_in=d_in)
    np.testing.assert_array_equal(Y, What.T)
