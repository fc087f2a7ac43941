"""The C-ABI library loads and exports every entry point include/gptq.h declares.

CPU only: no compute call is made; only host-side queries and the argument
checks that return before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")
LIB = os.path.join(ROOT, "post_weight_quantization_syrk_amd", "libgptq_mi355x.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq_[a-z0-9_]+)\s*\(", text)))


def _lib():
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    return ctypes.CDLL(LIB)


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("gptq_hessian_accumulate", "gptq_prepare_hinv", "gptq_quantize_layer", "gptq_pack"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_host_queries():
    from post_weight_quantization_syrk_amd import gptq
    if not os.path.exists(gptq.LIB_PATH):
        pytest.skip("library not built")
    assert gptq.lib().gptq_abi_version() == 100
    assert gptq.strerror(0) == "ok"
    assert "positive definite" in gptq.strerror(4)
    # workspace sizes: split-K partials, factorization scratch, working copies
    assert gptq.gptq_hessian_workspace(4096, 262144, gptq.GPTQ_BF16) > 0
    assert gptq.gptq_hessian_workspace(4096, 0, gptq.GPTQ_BF16) == 0
    assert gptq.gptq_prepare_workspace(4096) >= 2 * 4096 * 4096 * 4  # two fp32 d x d arrays
    assert gptq.gptq_quantize_workspace(4096, 4096) >= 2 * 4096 * 4096 * 4


def test_argument_errors_return_before_any_launch():
    from post_weight_quantization_syrk_amd import gptq
    if not os.path.exists(gptq.LIB_PATH):
        pytest.skip("library not built")
    L = gptq.lib()
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: every call below fails validation first
    # bad dtype / sizes
    assert L.gptq_hessian_accumulate(fake, 16, fake, 7, 10, 16, None, 0, None) == gptq.GPTQ_EINVAL
    assert L.gptq_hessian_accumulate(fake, 16, fake, 0, 10, 8, None, 0, None) == gptq.GPTQ_EINVAL
    assert L.gptq_hessian_accumulate(fake, 16, fake, 0, 10, 16, None, 0, None) == gptq.GPTQ_EINVAL  # no ws
    assert L.gptq_hessian_accumulate(None, 16, fake, 0, 10, 16, None, 0, None) == gptq.GPTQ_EINVAL
    assert L.gptq_hessian_accumulate(fake, 16, fake, 0, 0, 16, None, 0, None) == gptq.GPTQ_OK  # no-op
    # prepare: missing workspace, negative damping
    assert L.gptq_prepare_hinv(fake, 8, 0.01, fake, None, fake, None, 0, None) == gptq.GPTQ_EINVAL
    assert L.gptq_prepare_hinv(fake, 8, -1.0, fake, None, fake, fake, 1 << 20, None) == gptq.GPTQ_EINVAL
    # quantize: bits, group size, block
    q = L.gptq_quantize_layer
    args = lambda bits, g, sym, block, d_in=256: (fake, 0, 4, d_in, fake, None, bits, g, sym, block,
                                                   fake, fake, fake, None, None, 0, None)
    assert q(*args(5, 128, 0, 128)) == gptq.GPTQ_EINVAL
    assert q(*args(8, 128, 0, 128)) == gptq.GPTQ_EUNSUPPORTED
    assert q(*args(4, 48, 0, 128)) == gptq.GPTQ_EINVAL       # 48 does not divide 256
    assert q(*args(4, 16, 0, 128)) == gptq.GPTQ_EUNSUPPORTED  # divides, not implemented
    assert q(*args(4, 128, 0, 64)) == gptq.GPTQ_EUNSUPPORTED
    assert q(*args(4, 128, 2, 128)) == gptq.GPTQ_EINVAL
    assert q(*args(4, 128, 0, 128)) == gptq.GPTQ_EINVAL      # no workspace
    # pack
    assert L.gptq_pack(fake, fake, fake, 4, 256, 5, 128, 0, fake, fake, fake, None) == gptq.GPTQ_EINVAL
    assert L.gptq_pack(fake, fake, None, 4, 256, 4, 128, 0, fake, fake, None, None) == gptq.GPTQ_EINVAL
    # two-sided rounding: sizes, workspace, pointers
    r = L.gptq2d_round
    assert gptq.gptq2d_workspace(1024) == 2 * 1024 * 1024 * 8
    assert gptq.gptq2d_workspace(0) == 0 and gptq.gptq2d_workspace(40000) == 0
    assert r(fake, fake, fake, -1, fake, fake, 1 << 20, None) == gptq.GPTQ_EINVAL
    assert r(fake, fake, fake, 40000, fake, fake, 1 << 40, None) == gptq.GPTQ_EUNSUPPORTED
    assert r(fake, fake, fake, 0, fake, None, 0, None) == gptq.GPTQ_OK  # no-op
    assert r(fake, None, fake, 16, fake, fake, 1 << 20, None) == gptq.GPTQ_EINVAL
    assert r(fake, fake, fake, 16, fake, fake, 16, None) == gptq.GPTQ_EINVAL     # workspace too small
    assert r(fake, fake, fake, 16, fake, P(0x1010), 1 << 20, None) == gptq.GPTQ_EINVAL  # unaligned
    # activation ordering, permuted factorization and quantization
    assert L.gptq_act_order(fake, 0, 10, 8, 16, fake, None, fake, 1 << 20, None) == gptq.GPTQ_EINVAL  # ldx < d
    assert L.gptq_act_order(fake, 0, 10, 16, 16, None, None, fake, 1 << 20, None) == gptq.GPTQ_EINVAL
    assert L.gptq_act_order(fake, 0, 10, 16, 16, fake, None, fake, 8, None) == gptq.GPTQ_EINVAL
    assert L.gptq_prepare_hinv_perm(fake, 8, 0.01, None, fake, None, fake, None, 0, None) == gptq.GPTQ_EINVAL
    qp = L.gptq_quantize_layer_perm
    pargs = lambda static, bits=4, g=128: (fake, 0, 4, 256, fake, None, fake, static, bits, g, 0, 128,
                                           fake, fake, fake, None, None, fake, 1 << 30, None)
    assert qp(*pargs(2)) == gptq.GPTQ_EINVAL
    assert qp(*pargs(0, bits=8)) == gptq.GPTQ_EUNSUPPORTED
    assert qp(*pargs(0, g=48)) == gptq.GPTQ_EINVAL
    assert gptq.gptq_quantize_perm_workspace(4096, 4096) == gptq.gptq_quantize_workspace(4096, 4096) + 4096 * 4096
    assert gptq.gptq_act_order_workspace(4096, 262144) >= 256 * 4096 * 8
    # dequantized product
    w = L.gptq_w4a16_matmul
    assert w(fake, 4, 256, fake, fake, fake, 8, 200, 128, 0, fake, None) == gptq.GPTQ_EINVAL      # 128 does not divide 200
    assert w(fake, 4, 192, fake, fake, fake, 8, 192, 64, 0, fake, None) == gptq.GPTQ_EUNSUPPORTED  # d_in % 128
    assert w(fake, 4, 250, fake, fake, fake, 8, 256, 128, 0, fake, None) == gptq.GPTQ_EINVAL      # ldx < d_in
    assert w(fake, 4, 260, fake, fake, fake, 8, 256, 128, 0, fake, None) == gptq.GPTQ_EINVAL      # ldx % 8
    assert w(fake, 4, 256, fake, fake, None, 8, 256, 128, 0, fake, None) == gptq.GPTQ_EINVAL      # zeros needed
    assert w(P(0x1008), 4, 256, fake, fake, fake, 8, 256, 128, 0, fake, None) == gptq.GPTQ_EINVAL  # unaligned X
    assert w(fake, 0, 256, fake, fake, fake, 8, 256, 128, 0, fake, None) == gptq.GPTQ_OK         # no rows
    # layers sharing one Hessian
    ql = L.gptq_quantize_layers
    one = (P * 1)(fake)
    rows = (ctypes.c_int64 * 1)(4)
    assert ql(one, rows, 0, 0, 256, fake, None, 4, 128, 0, 128, fake, fake, fake, None, fake, 1 << 30, None) == gptq.GPTQ_EINVAL
    assert ql(one, rows, 1, 0, 256, fake, None, 5, 128, 0, 128, fake, fake, fake, None, fake, 1 << 30, None) == gptq.GPTQ_EINVAL
    assert ql(one, rows, 1, 0, 256, fake, None, 4, 128, 0, 64, fake, fake, fake, None, fake, 1 << 30, None) == gptq.GPTQ_EUNSUPPORTED
    assert ql(one, rows, 1, 0, 256, fake, None, 4, 128, 0, 128, fake, fake, fake, None, fake, 16, None) == gptq.GPTQ_EINVAL
    zero_rows = (ctypes.c_int64 * 1)(0)
    assert ql(one, zero_rows, 1, 0, 256, fake, None, 4, 128, 0, 128, fake, fake, fake, None, None, 0, None) == gptq.GPTQ_OK
