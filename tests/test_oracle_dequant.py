"""Pins of the dequantized-product oracle ([P1] 阶段三; [P5] 存储代价).  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def _packed(bits, g, sym, d_out=6, d_in=64, seed=0):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((d_out, d_in)) * 0.05
    r = oracle.rtn(W, bits=bits, group_size=g, sym=sym)
    qw = oracle.pack_rows(r["codes"], bits)
    s16 = oracle.fp16_bits(r["scales"])
    z16 = None if sym else oracle.fp16_bits(r["zeros"])
    return r, qw, s16, z16


@pytest.mark.parametrize("bits,g,sym", [(4, 16, False), (4, -1, True), (3, 32, False),
                                        (2, 16, True), (4, 32, True)])
def test_round_trip_reproduces_the_quantizers_w_hat(bits, g, sym):
    # pack -> dequantize gives back exactly the W_hat the quantizer formed
    r, qw, s16, z16 = _packed(bits, g, sym)
    What = oracle.dequantize(qw, s16, z16, bits=bits, group_size=g, sym=sym, d_in=64)
    np.testing.assert_array_equal(What, r["What"])


def test_hand_example():
    # one row, 4-bit, one group of 8: codes 0..7 in one word, scale 0.5, zero 3
    codes = np.arange(8, dtype=np.uint8)[None, :]
    qw = oracle.pack_rows(codes, 4)
    assert int(qw[0, 0]) == 0x76543210
    s16 = oracle.fp16_bits(np.array([[0.5]]))
    z16 = oracle.fp16_bits(np.array([[3.0]]))
    What = oracle.dequantize(qw, s16, z16, bits=4, group_size=8, sym=False, d_in=8)
    np.testing.assert_array_equal(What[0], 0.5 * (np.arange(8) - 3.0))
    X = np.zeros((2, 8))
    X[0, 2] = 1.0
    X[1] = 1.0
    Y = oracle.dequant_matmul(X, qw, s16, z16, bits=4, group_size=8, sym=False)
    np.testing.assert_array_equal(Y[:, 0], [0.5 * (2 - 3), 0.5 * (28 - 24)])


def test_product_by_brute_force():
    r, qw, s16, z16 = _packed(4, 16, False, d_out=5, d_in=32, seed=3)
    X = np.random.default_rng(4).standard_normal((3, 32))
    Y = oracle.dequant_matmul(X, qw, s16, z16, bits=4, group_size=16, sym=False)
    What = r["What"]
    for m in range(3):
        for n in range(5):
            assert abs(Y[m, n] - sum(X[m, k] * What[n, k] for k in range(32))) <= 1e-12


def test_planted_mistake_fails():
    # adding the zero instead of subtracting it breaks the round trip
    r, qw, s16, z16 = _packed(4, 16, False)
    q = oracle.unpack_rows(qw, 4, 64).astype(np.float64)
    s = oracle.dequant_gemm.f16_bits_to_f64(s16)
    z = oracle.dequant_gemm.f16_bits_to_f64(z16)
    g = np.arange(64) // 16
    assert not np.array_equal(s[:, g] * (q + z[:, g]), r["What"])
