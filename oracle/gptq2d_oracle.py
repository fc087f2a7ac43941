"""Two-sided adaptive rounding (reference side), after [P2].

TEST INFRASTRUCTURE ONLY (see the package docstring).

Problem ([P2] 方法, 核心洞察): round a real n x n matrix Y to an integer matrix Z
so that the error is small in the metric that puts a fixed nonsingular basis on
each side.  Reading taken here (the page gives no formula): with upper
triangular bases R_L, R_R of positive diagonal, the metric is
    || R_L (Y - Z) R_R^T ||_F^2 = vec(E)^T (R_R^T R_R  kron  R_L^T R_L) vec(E),
vec() stacking columns.  The Gram is the Kronecker product the page names, and
its upper triangular factor is M = R_R kron R_L.

* ``two_sided_quartic``: the vectorized one-sided method ([P2] 问题背景: the
  Kronecker Gram handed to the one-dimensional algorithm, O(n^4)): Babai's
  nearest plane on the triangular basis M, last coordinate first.
* ``two_sided_antidiagonal``: the anti-diagonal schedule ([P2] 方法 steps 1-3):
  entry (i, j) depends only on entries (i', j') with i' >= i and j' >= j, so
  all entries with i + j = s are independent and the anti-diagonals are taken
  from s = 2n-2 down to 0.  Errors are carried through the two triangular
  factors with one running array P, P[k, j] = sum_{j' >= j} e[k, j'] R_R[j, j'],
  which costs O(n) per entry, O(n^3) in all.

Reading of [P2] 方法 step 1 ("从右上角到左下角"): both corners lie on the same
anti-diagonal, so the phrase is taken as the direction along one anti-diagonal,
which does not matter because its entries are independent.
"""
from __future__ import annotations

import numpy as np


def _check(Y, RL, RR):
    Y = np.asarray(Y, np.float64)
    RL = np.triu(np.asarray(RL, np.float64))
    RR = np.triu(np.asarray(RR, np.float64))
    n = Y.shape[0]
    if Y.shape != (n, n) or RL.shape != (n, n) or RR.shape != (n, n):
        raise ValueError("square n x n inputs expected")
    if np.any(np.diag(RL) <= 0) or np.any(np.diag(RR) <= 0):
        raise ValueError("bases need a positive diagonal")
    return Y, RL, RR, n


def two_sided_quartic(Y, RL, RR) -> np.ndarray:
    """Nearest plane on M = R_R kron R_L (column-major vec); O(n^4) time and memory."""
    Y, RL, RR, n = _check(Y, RL, RR)
    M = np.kron(RR, RL)
    y = Y.reshape(-1, order="F")
    t = M @ y
    N = n * n
    z = np.zeros(N)
    for m in range(N - 1, -1, -1):
        acc = t[m] - M[m, m + 1:] @ z[m + 1:]
        z[m] = np.rint(acc / M[m, m])
    return z.reshape((n, n), order="F")


def two_sided_antidiagonal(Y, RL, RR) -> np.ndarray:
    """Anti-diagonal schedule, O(n^3); every anti-diagonal handled as one vector step."""
    Y, RL, RR, n = _check(Y, RL, RR)
    Z = np.zeros((n, n))
    P = np.zeros((n, n))
    dL = np.diag(RL)
    dR = np.diag(RR)
    for s in range(2 * n - 2, -1, -1):
        i = np.arange(max(0, s - n + 1), min(s, n - 1) + 1)
        j = s - i
        # S_ij = sum_{k >= i} R_L[i, k] P[k, j]   (P[i, j] holds no own-entry term yet)
        S = np.array([RL[ii, ii:] @ P[ii:, jj] for ii, jj in zip(i, j)])
        z = np.rint(Y[i, j] + S / (dL[i] * dR[j]))
        Z[i, j] = z
        e = Y[i, j] - z
        # P[i, 0..j] += e_ij * R_R[0..j, j]; rows i are distinct on one anti-diagonal
        for ii, jj, ee in zip(i, j, e):
            P[ii, :jj + 1] += ee * RR[:jj + 1, jj]
    return Z
