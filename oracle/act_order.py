"""Activation ordering and static groups, float64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P1] "GPTQ：基于近似二阶信息的大模型权重量化", GPTQ 的高级技巧:
  * 激活排序（desc_act）: the columns of W are not taken in their natural
    order but reordered by the sum of the absolute values of their input
    activations, so that the columns with less effect on the output are
    quantized first and the error feedback lands on the more sensitive ones.
    Reading taken here: influence of column c = sum_t |x_t,c| over the
    calibration tokens, and the processing order is ascending in it (least
    influential first), ties by column index.  (The flag's name says
    "descending"; the page's sentence fixes the direction, and it is what is
    followed.)
  * 静态与动态分组: with static groups the group size is fixed at quantization
    time and inference looks the parameters up simply.  Reading taken here:
    the groups stay the natural runs of group_size columns (g_idx[c] = c // g)
    and their parameters are set from the original weights before any error
    feedback, so a permuted processing order does not scatter a group.  With
    dynamic groups (the default) a group is a run of group_size consecutive
    columns in processing order, parameters set at its first column from the
    current values, as in the natural-order method; g_idx[perm[k]] = k // g.

The method itself is unchanged: W's columns and H's rows and columns are
permuted, the one-sided path runs on the permuted problem, and codes, W_hat
and the scaled errors are mapped back to natural column order.
"""
from __future__ import annotations

import numpy as np

from .gptq_oracle import column_loop, gptq, group_params, maxq_for, prepare, quantize_values


def activation_order(chunks) -> np.ndarray:
    """perm[k] = the k-th column to quantize: ascending sum_t |x_t,c|, ties by index."""
    a = None
    for x in chunks:
        s = np.abs(np.asarray(x, dtype=np.float64)).sum(axis=0)
        a = s if a is None else a + s
    return np.argsort(a, kind="stable"), a


def _lower_to_symmetric(H0):
    L = np.tril(np.asarray(H0, dtype=np.float64))
    return L + np.tril(L, -1).T


def gptq_ordered(W, H0, perm, *, damp=0.01, bits=4, group_size=128, sym=False, block=None,
                 static_groups=False) -> dict:
    """GPTQ with columns processed in the order ``perm``.

    H0 is the undamped Hessian (lower triangle authoritative).  Returns
    dict(codes, scales, zeros, g_idx, What, delta, loss_damped, U (of the
    permuted problem), dead (natural order)).  scales/zeros are indexed by
    group: natural groups when static, processing-order groups when dynamic.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    d_out, d_in = W.shape
    perm = np.asarray(perm, dtype=np.int64)
    if sorted(perm.tolist()) != list(range(d_in)):
        raise ValueError("perm must be a permutation of the columns")
    Hs = _lower_to_symmetric(H0)
    dead = np.diag(Hs) == 0.0
    W[:, dead] = 0.0
    P = prepare(Hs[np.ix_(perm, perm)], damp)
    U = P["U"]
    Wp = W[:, perm]
    G = d_in if group_size in (-1, None) else int(group_size)
    g_idx = np.zeros(d_in, dtype=np.int64)
    if not static_groups or G == d_in:
        r = gptq(Wp, U, P["dead"], bits=bits, group_size=group_size, sym=sym, block=block)
        codes_p, What_p, delta_p = r["codes"], r["What"], r["delta"]
        scales, zeros = r["scales"], r["zeros"]
        raw_q_p, raw_scales, raw_zeros = r["raw_q"], r["raw_scales"], r["raw_zeros"]
        g_idx[perm] = np.arange(d_in) // G
    else:
        maxq = maxq_for(bits)
        ng = d_in // G
        scales = np.zeros((d_out, ng))
        zeros = np.zeros((d_out, ng))
        raw_scales = np.zeros((d_out, ng))
        raw_zeros = np.zeros((d_out, ng))
        for g in range(ng):
            scales[:, g], zeros[:, g], raw_scales[:, g], raw_zeros[:, g] = group_params(
                W[:, g * G:(g + 1) * G], bits, sym, with_raw=True)
        codes_p = np.zeros((d_out, d_in), dtype=np.uint8)
        raw_q_p = np.zeros((d_out, d_in))

        def qcol(k, Wc):
            g = perm[k] // G
            q, wh = quantize_values(Wc[:, k], scales[:, g], zeros[:, g], maxq)
            codes_p[:, k] = q.astype(np.uint8)
            raw_q_p[:, k] = Wc[:, k] / scales[:, g]
            return wh

        _, What_p, delta_p = column_loop(Wp, U, qcol, block=block)
        g_idx[:] = np.arange(d_in) // G
    codes = np.empty_like(codes_p)
    What = np.empty_like(What_p)
    delta = np.empty_like(delta_p)
    codes[:, perm] = codes_p
    What[:, perm] = What_p
    delta[:, perm] = delta_p
    # the *_p entries are in processing order (column k = natural column
    # perm[k]); raw_q_p is the unrounded quotient w / scale of each code
    return dict(codes=codes, scales=scales, zeros=zeros, g_idx=g_idx, What=What, delta=delta,
                loss_damped=np.sum(delta * delta, axis=1), U=U, dead=dead,
                H_damped_perm=P["H"], codes_p=codes_p, What_p=What_p, raw_q_p=raw_q_p,
                raw_scales=raw_scales, raw_zeros=raw_zeros)
