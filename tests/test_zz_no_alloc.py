"""The allocation-free Hessian entry point against the regular one, through the
C ABI: bit-identical where the split count is the same, within the Hessian
tolerance where the fixed scratch caps it; two calls in a row, the second
smaller; sizes beyond the fixed array rejected before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import DEV, dev_bf16, dev_f32
from parity import h_rel_error
from post_weight_quantization_syrk_amd import gptq, synth

pytestmark = pytest.mark.gpu


def _x(n, d, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d), dtype=np.float32) * np.exp(rng.standard_normal(d)).astype(
        np.float32)
    return dev_bf16(synth.f32_to_bf16_bits(x)) if dtype == "bf16" else dev_f32(x)


def _both(X, d):
    Ha = torch.zeros((d, d), dtype=torch.float32, device=DEV)
    Hb = torch.zeros((d, d), dtype=torch.float32, device=DEV)
    gptq.gptq_hessian_accumulate(Ha, X)
    gptq.gptq_hessian_accumulate_noalloc(Hb, X)
    torch.cuda.synchronize()
    return Ha.cpu().numpy(), Hb.cpu().numpy()


def test_noalloc_matches_regular_two_calls_second_smaller():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    assert gptq.gptq_noalloc_scratch_bytes() == 64 << 20
    # first call: 640 wide, 5000 tokens (split count unchanged by the cap)
    print("[noalloc] bf16 5000 x 640", flush=True)
    a, b = _both(_x(5000, 640, "bf16", 1), 640)
    np.testing.assert_array_equal(np.tril(a), np.tril(b))
    # second call, smaller: 300 wide, 1000 tokens, on the same scratch
    print("[noalloc] bf16 1000 x 300", flush=True)
    a, b = _both(_x(1000, 300, "bf16", 2), 300)
    np.testing.assert_array_equal(np.tril(a), np.tril(b))


def test_noalloc_capped_splits_and_fp32():
    # 4096 wide: one 256-wide split's partial tiles take 34 MiB, so the
    # 64 MiB array holds one split where the regular call uses several:
    # the same sums in another order, within the Hessian tolerance
    print("[noalloc] bf16 32768 x 4096 (capped splits)", flush=True)
    a, b = _both(_x(32768, 4096, "bf16", 3), 4096)
    err = h_rel_error(b, a)
    print(f"[noalloc] capped: rel Frobenius difference {err:.2e}", flush=True)
    assert err <= 1e-5
    print("[noalloc] fp32 3000 x 513", flush=True)
    a, b = _both(_x(3000, 513, "f32", 4), 513)
    np.testing.assert_array_equal(np.tril(a), np.tril(b))


def test_noalloc_rejects_sizes_beyond_the_array():
    d = 5633  # 23 tiles of 256: one split's partials exceed 64 MiB
    X = torch.zeros((16, d), dtype=torch.bfloat16, device=DEV)
    H = torch.zeros((d, d), dtype=torch.float32, device=DEV)
    with pytest.raises(gptq.GPTQError) as e:
        gptq.gptq_hessian_accumulate_noalloc(H, X)
    assert e.value.status == gptq.GPTQ_EUNSUPPORTED
    # d = 5632 still fits
    Xs = _x(64, 5632, "bf16", 5)
    Hs = torch.zeros((5632, 5632), dtype=torch.float32, device=DEV)
    gptq.gptq_hessian_accumulate_noalloc(Hs, Xs)
    torch.cuda.synchronize()
    ref = torch.zeros_like(Hs)
    gptq.gptq_hessian_accumulate(ref, Xs)
    torch.cuda.synchronize()
    assert h_rel_error(Hs.cpu().numpy(), ref.cpu().numpy()) <= 1e-5
