"""Float64 reference for one-sided GPTQ on one linear layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the
product path, shares no code with it.

What it computes, step by step, in the order of [P1] 阶段一/阶段二/阶段三:

  1. Hessian        H0 = 2 * sum_t x_t x_t^T over calibration tokens  ([P1] 阶段一).
  2. Dead channels  diag(H0)_i == 0  ->  H_ii = 1 and W[:, i] = 0 (reading: the
                    pages are silent; such an input never reaches the output).
  3. Damping        H = H0 + lambda*I, lambda = damp * mean(diag H)  ([P1] 阶段一
                    gives "2X^T X + lambda I" without a value; damp = 0.01).
  4. Cholesky       H = L L^T  ([P1] 阶段一 step 2, 伪代码逻辑).
  5. Upper factor   U upper triangular with U^T U = H^{-1}, obtained literally:
                    Hinv = L^-T L^-1, then U = chol(Hinv)^T.
  6. Column loop    columns in natural order ([P1] 阶段二 "贪婪顺序"); rows
                    independent ([P4] "row-wise quantization").  At each
                    group's first column the group's *current* values set its
                    scale and zero ([P1] 对称与仿射量化/分组量化, [P5] 小 group 买到了什么);
                    each column is rounded, q = clamp(round(w/s) + z, 0, maxq),
                    w_hat = s (q - z) ([P1] 对称与仿射量化, [P5] the 0..15 grid);
                    its scaled error delta = (w - w_hat)/U_jj is fed into the
                    later columns, w_k -= delta * U_jk ([P1] 量化误差与补偿,
                    核心思想 "权重量化补偿").
  7. Lazy batching  the same arithmetic with the feedback to columns past the
                    current block of B columns deferred to one matrix product
                    per block ([P1] 阶段二 "懒惰更新").

Readings where the pages are silent (all listed in the design notes too):
  * The range of an asymmetric group always contains 0 ([P5]: the zero point
    is the integer that stands for 0, so it must lie on the grid).
  * Asymmetric step = (hi - lo)/maxq ([P5]: "range divided by 15" at 4 bits);
    symmetric step = 2*max|v|/maxq with offset (maxq+1)/2 (the [P5] worked
    example's 0.067 for a lone 0.5 outlier is 2*0.5/15).
  * The step is rounded once, from float64, to IEEE binary16 before use, so
    dequantizing the stored 16-bit scale reproduces the value that drove the
    error feedback ([P1] 支持的数据类型, [P5] 存储代价: 16-bit scales).
  * round() is to the nearest integer of the exact quotient, ties to even.
  * A group whose range is zero (or whose step rounds to 0 in binary16) gets
    step 1; every value in it then maps to the zero point.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg.lapack as lapack


class NotSPD(ValueError):
    """Cholesky broke down; ``pivot`` is the 1-based index of the failing pivot."""

    def __init__(self, pivot: int):
        super().__init__(f"matrix is not positive definite (pivot {pivot})")
        self.pivot = int(pivot)


def maxq_for(bits: int) -> int:
    """Largest code: 2^b - 1 ([P5]: 16 / 8 / 4 levels at 4 / 3 / 2 bits)."""
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    return (1 << bits) - 1


def fp16_rne(x) -> np.ndarray:
    """Round float64 values once to IEEE binary16 (nearest, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# 1. Hessian  ([P1] 阶段一: H = 2 X^T X)
# ---------------------------------------------------------------------------
def hessian(chunks, d: int | None = None) -> np.ndarray:
    """H0 = 2 * sum over tokens of x x^T, accumulated in float64 chunk by chunk.

    ``chunks`` yields float64 arrays [tokens, d] holding exactly the values the
    caller feeds the layer (bf16/fp32 inputs widen exactly).  Not normalised by
    the token count: the damping is relative, so the result does not depend on
    it.
    """
    H = None
    for xc in chunks:
        xc = np.asarray(xc, dtype=np.float64)
        if not np.all(np.isfinite(xc)):
            raise ValueError("non-finite calibration input")
        if H is None:
            H = np.zeros((xc.shape[1], xc.shape[1]))
        H += 2.0 * (xc.T @ xc)
    if H is None:
        H = np.zeros((d, d))
    return H


def hessian_entry(x: np.ndarray, i: int, j: int) -> float:
    """One entry of H0 computed on its own: 2 * sum_t x[t, i] * x[t, j]."""
    return 2.0 * float(np.dot(np.asarray(x[:, i], np.float64), np.asarray(x[:, j], np.float64)))


# ---------------------------------------------------------------------------
# 2-5. Dead channels, damping, Cholesky, upper factor of the inverse
# ---------------------------------------------------------------------------
def _symmetrize_lower(H: np.ndarray) -> np.ndarray:
    """The lower triangle is authoritative; mirror it into the upper one."""
    lo = np.tril(H)
    return lo + np.tril(H, -1).T


def _chol_lower(A: np.ndarray) -> np.ndarray:
    c, info = lapack.dpotrf(A, lower=1, clean=1)
    if info > 0:
        raise NotSPD(info)
    if info < 0:
        raise ValueError("dpotrf argument error")
    return c


def prepare(H0: np.ndarray, damp: float = 0.01) -> dict:
    """Dead-channel fix, damping, Cholesky and the upper factor U of H^-1.

    Returns dict(dead, H (damped), lam, L, U).  Raises NotSPD on breakdown.
    """
    H = _symmetrize_lower(np.asarray(H0, dtype=np.float64))
    if not np.all(np.isfinite(H)):
        raise ValueError("non-finite Hessian")
    d = H.shape[0]
    dead = np.diag(H) == 0.0
    H[dead, dead] = 1.0
    lam = damp * float(np.mean(np.diag(H))) if d else 0.0
    H[np.arange(d), np.arange(d)] += lam
    L = _chol_lower(H)
    Linv, info = lapack.dtrtri(L, lower=1)
    if info != 0:
        raise NotSPD(info)
    Hinv = Linv.T @ Linv
    Hinv = _symmetrize_lower(Hinv)
    # upper Cholesky factor of Hinv: Hinv = U^T U
    U, info = lapack.dpotrf(Hinv, lower=0, clean=1)
    if info > 0:
        raise NotSPD(info)
    return dict(dead=dead, H=H, lam=lam, L=L, U=np.triu(U))


def reversed_route_U(H: np.ndarray) -> np.ndarray:
    """U from the reversed factorization H = V V^T (V upper), U = V^{-1}.

    With J the order-reversing permutation, V = J chol(J H J) J.  Used only to
    check that the literal route above gives the same (unique) factor.
    """
    H = np.asarray(H, dtype=np.float64)
    J = np.eye(H.shape[0])[::-1]
    Lr = _chol_lower(J @ H @ J)
    V = J @ Lr @ J
    Vinv, info = lapack.dtrtri(V, lower=0)
    if info != 0:
        raise NotSPD(info)
    return np.triu(Vinv)


# ---------------------------------------------------------------------------
# 6. Quantizer: group parameters and rounding
# ---------------------------------------------------------------------------
def group_params(v: np.ndarray, bits: int, sym: bool, with_raw: bool = False):
    """Scale (binary16 value) and integer zero of each row of ``v`` [rows, G].

    With ``with_raw`` also returns the unrounded step (hi-lo)/maxq or
    2 max|v|/maxq and the unrounded zero -lo/scale, for reporting how close a
    value sat to a rounding boundary.
    """
    maxq = maxq_for(bits)
    v = np.asarray(v, dtype=np.float64)
    rows = v.shape[0]
    scale = np.ones(rows)
    if sym:
        zero = np.full(rows, float((maxq + 1) // 2))
        amax = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(rows)
        raw = 2.0 * amax / maxq
        s16 = fp16_rne(raw)
        ok = (amax > 0) & (s16 > 0)
        scale[ok] = s16[ok]
        if with_raw:
            return scale, zero, raw, zero.copy()
        return scale, zero
    lo = np.minimum(0.0, np.min(v, axis=1)) if v.shape[1] else np.zeros(rows)
    hi = np.maximum(0.0, np.max(v, axis=1)) if v.shape[1] else np.zeros(rows)
    raw = (hi - lo) / maxq
    s16 = fp16_rne(raw)
    ok = (hi > lo) & (s16 > 0)
    scale[ok] = s16[ok]
    zero = np.zeros(rows)
    zraw = -lo / scale
    zero[ok] = np.clip(np.rint(zraw[ok]), 0, maxq)
    if with_raw:
        return scale, zero, raw, zraw
    return scale, zero


def quantize_values(w: np.ndarray, scale: np.ndarray, zero: np.ndarray, maxq: int):
    """q = clamp(round(w/s) + z, 0, maxq); w_hat = s (q - z)."""
    q = np.clip(np.rint(w / scale) + zero, 0, maxq)
    return q, scale * (q - zero)


# ---------------------------------------------------------------------------
# 6-7. Column loop with error feedback, sequential or lazily batched
# ---------------------------------------------------------------------------
def column_loop(W: np.ndarray, U: np.ndarray, quantize_col, block: int | None = None):
    """Greedy column-by-column rounding with error feedback through U.

    ``quantize_col(j, Wc)`` returns the rounded values of column j given the
    current working matrix ``Wc`` (it may look at later columns, e.g. to set a
    group's parameters).  With ``block`` None every error is applied to every
    later column at once; with ``block`` = B the feedback to columns past the
    current block is deferred and applied as  W[:, rest] -= Err @ U[blk, rest].
    Returns (Wc_final, What, delta).
    """
    Wc = np.array(W, dtype=np.float64, copy=True)
    d_out, d_in = Wc.shape
    What = np.zeros_like(Wc)
    delta = np.zeros_like(Wc)
    B = d_in if block is None else int(block)
    for b0 in range(0, d_in, B):
        b1 = min(b0 + B, d_in)
        end = d_in if block is None else b1
        for j in range(b0, b1):
            wh = quantize_col(j, Wc)
            What[:, j] = wh
            dj = (Wc[:, j] - wh) / U[j, j]
            delta[:, j] = dj
            if j + 1 < end:
                Wc[:, j + 1:end] -= np.outer(dj, U[j, j + 1:end])
        if block is not None and b1 < d_in:
            Wc[:, b1:] -= delta[:, b0:b1] @ U[b0:b1, b1:]
    return Wc, What, delta


def gptq(W, U, dead=None, *, bits=4, group_size=128, sym=False, block=None):
    """GPTQ on one layer.  W [d_out, d_in] (any float), U from ``prepare``.

    Returns dict(codes uint8, scales, zeros [d_out, n_groups], What, delta,
    loss_damped [d_out] = sum_j delta_j^2).
    """
    W = np.array(W, dtype=np.float64, copy=True)
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weights")
    d_out, d_in = W.shape
    maxq = maxq_for(bits)
    G = d_in if group_size in (-1, None) else int(group_size)
    if d_in % G:
        raise ValueError("d_in must be a multiple of group_size")
    if block is not None and group_size not in (-1, None) and block % G:
        raise ValueError("block must be a multiple of group_size")
    if dead is not None:
        W[:, np.asarray(dead, dtype=bool)] = 0.0
    ng = d_in // G
    scales = np.zeros((d_out, ng))
    zeros = np.zeros((d_out, ng))
    raw_scales = np.zeros((d_out, ng))
    raw_zeros = np.zeros((d_out, ng))
    raw_q = np.zeros((d_out, d_in))
    codes = np.zeros((d_out, d_in), dtype=np.uint8)
    cur = {}

    def qcol(j, Wc):
        if j % G == 0:
            s, z, rs, rz = group_params(Wc[:, j:j + G], bits, sym, with_raw=True)
            scales[:, j // G] = s
            zeros[:, j // G] = z
            raw_scales[:, j // G] = rs
            raw_zeros[:, j // G] = rz
            cur["s"], cur["z"] = s, z
        q, wh = quantize_values(Wc[:, j], cur["s"], cur["z"], maxq)
        codes[:, j] = q.astype(np.uint8)
        raw_q[:, j] = Wc[:, j] / cur["s"]
        return wh

    _, What, delta = column_loop(W, U, qcol, block=block)
    return dict(codes=codes, scales=scales, zeros=zeros, What=What, delta=delta,
                loss_damped=np.sum(delta * delta, axis=1), raw_scales=raw_scales,
                raw_zeros=raw_zeros, raw_q=raw_q)


def rtn(W, *, bits=4, group_size=128, sym=False):
    """Round-to-nearest baseline: every group rounded on its own values, no feedback."""
    W = np.asarray(W, dtype=np.float64)
    d_out, d_in = W.shape
    maxq = maxq_for(bits)
    G = d_in if group_size in (-1, None) else int(group_size)
    codes = np.zeros((d_out, d_in), dtype=np.uint8)
    What = np.zeros_like(W)
    scales = np.zeros((d_out, d_in // G))
    zeros = np.zeros_like(scales)
    for g in range(d_in // G):
        sl = slice(g * G, (g + 1) * G)
        s, z = group_params(W[:, sl], bits, sym)
        q = np.clip(np.rint(W[:, sl] / s[:, None]) + z[:, None], 0, maxq)
        codes[:, sl] = q.astype(np.uint8)
        What[:, sl] = s[:, None] * (q - z[:, None])
        scales[:, g], zeros[:, g] = s, z
    return dict(codes=codes, scales=scales, zeros=zeros, What=What)


def layer_loss(W, What, H0) -> float:
    """tr((W - What) H0 (W - What)^T) with the undamped H0.

    [P1] 阶段一 writes the layer error as ||WX - What X||_F^2 with X [n, d_in];
    dimensionally it is ||(W - What) X^T||_F^2, which equals this trace / 2.
    """
    E = np.asarray(W, np.float64) - np.asarray(What, np.float64)
    return float(np.sum((E @ np.asarray(H0, np.float64)) * E))
