"""Pins of the activation-ordering oracle ([P1] "GPTQ：基于近似二阶信息的大模型权重量化",
GPTQ 的高级技巧: 激活排序（desc_act）and 静态与动态分组).  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def _layer(d_out=12, d_in=64, seed=0):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((d_out, d_in)) * 0.05
    X = rng.standard_normal((200, d_in)) * np.exp(rng.standard_normal(d_in))
    return W, X, oracle.hessian([X])


def test_order_hand_example():
    # sum |x| per column: [3, 4, 1, 3] -> ascending, ties by index: 2, 0, 3, 1
    X = np.array([[1.0, -3.0, 0.5, 2.0], [2.0, 1.0, -0.5, -1.0]])
    perm, a = oracle.activation_order([X[:1], X[1:]])
    np.testing.assert_array_equal(a, [3.0, 4.0, 1.0, 3.0])
    np.testing.assert_array_equal(perm, [2, 0, 3, 1])


def test_identity_order_is_the_plain_path():
    W, X, H0 = _layer()
    ref = oracle.gptq(W, oracle.prepare(H0)["U"], bits=4, group_size=16, block=32)
    got = oracle.gptq_ordered(W, H0, np.arange(64), bits=4, group_size=16, block=32)
    np.testing.assert_array_equal(got["codes"], ref["codes"])
    np.testing.assert_array_equal(got["scales"], ref["scales"])
    np.testing.assert_array_equal(got["g_idx"], np.arange(64) // 16)


@pytest.mark.parametrize("sym", [False, True])
def test_diagonal_hessian_static_groups_are_rtn_for_any_order(sym):
    # no feedback between columns: static groups must give round-to-nearest of W
    # with its natural groups, whatever the processing order
    W, _, _ = _layer(seed=3)
    H0 = np.diag(np.linspace(1.0, 4.0, 64))
    perm = np.random.default_rng(9).permutation(64)
    got = oracle.gptq_ordered(W, H0, perm, bits=3, group_size=16, sym=sym, static_groups=True)
    ref = oracle.rtn(W, bits=3, group_size=16, sym=sym)
    np.testing.assert_array_equal(got["codes"], ref["codes"])
    np.testing.assert_array_equal(got["scales"], ref["scales"])
    np.testing.assert_array_equal(got["zeros"], ref["zeros"])
    np.testing.assert_array_equal(got["g_idx"], np.arange(64) // 16)


def test_diagonal_hessian_dynamic_groups_follow_processing_order():
    W, _, _ = _layer(seed=4)
    H0 = np.diag(np.linspace(1.0, 4.0, 64))
    perm = np.random.default_rng(10).permutation(64)
    got = oracle.gptq_ordered(W, H0, perm, bits=4, group_size=16)
    ref = oracle.rtn(W[:, perm], bits=4, group_size=16)
    np.testing.assert_array_equal(got["codes"][:, perm], ref["codes"])
    np.testing.assert_array_equal(got["scales"], ref["scales"])
    g = np.empty(64, dtype=np.int64)
    g[perm] = np.arange(64) // 16
    np.testing.assert_array_equal(got["g_idx"], g)


def test_static_parameters_come_from_the_original_weights():
    W, X, H0 = _layer(seed=5)
    perm, _ = oracle.activation_order([X])
    got = oracle.gptq_ordered(W, H0, perm, bits=4, group_size=16, static_groups=True)
    ref = oracle.rtn(W, bits=4, group_size=16)
    np.testing.assert_array_equal(got["scales"], ref["scales"])
    np.testing.assert_array_equal(got["zeros"], ref["zeros"])
    # every code dequantizes with its column's group parameters
    g = got["g_idx"]
    What = got["scales"][:, g] * (got["codes"] - got["zeros"][:, g])
    np.testing.assert_allclose(What, got["What"], rtol=0, atol=0)


def test_loss_identity_in_natural_order():
    # sum_j delta_j^2 = (w - w_hat) H (w - w_hat)^T with the damped H in natural order
    W, X, H0 = _layer(seed=6)
    perm, _ = oracle.activation_order([X])
    for static in (False, True):
        r = oracle.gptq_ordered(W, H0, perm, bits=4, group_size=16, static_groups=static)
        inv = np.argsort(perm)
        Hd = r["H_damped_perm"][np.ix_(inv, inv)]
        E = W - r["What"]
        np.testing.assert_allclose(np.einsum("ij,jk,ik->i", E, Hd, E), r["loss_damped"],
                                   rtol=1e-9)


def test_planted_mistakes_fail_a_pin():
    # descending order breaks the hand example; skipping the un-permute breaks
    # the diagonal-Hessian pin
    X = np.array([[1.0, -3.0, 0.5, 2.0], [2.0, 1.0, -0.5, -1.0]])
    a = np.abs(X).sum(axis=0)
    assert not np.array_equal(np.argsort(-a, kind="stable"), oracle.activation_order([X])[0])
    W, _, _ = _layer(seed=3)
    H0 = np.diag(np.linspace(1.0, 4.0, 64))
    perm = np.random.default_rng(9).permutation(64)
    got = oracle.gptq_ordered(W, H0, perm, bits=3, group_size=16, static_groups=True)
    assert not np.array_equal(got["codes"][:, perm], oracle.rtn(W, bits=3, group_size=16)["codes"])


def test_dead_columns_and_order():
    W, X, H0 = _layer(seed=7)
    X[:, [5, 40]] = 0.0
    H0 = oracle.hessian([X])
    perm, a = oracle.activation_order([X])
    assert set(perm[:2].tolist()) == {5, 40}   # zero influence: quantized first
    r = oracle.gptq_ordered(W, H0, perm, bits=4, group_size=16, static_groups=True)
    assert r["dead"][5] and r["dead"][40]
    assert np.all(r["What"][:, [5, 40]] == 0.0)
