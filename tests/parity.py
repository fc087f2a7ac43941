"""Comparison helpers between the HIP path's outputs and the oracle's.

Tolerances (GPU vs float64 oracle on the same seeded inputs):
  * Hessian: ||H_gpu - H_ref||_F / ||H_ref||_F <= 1e-4 (lower triangle).
  * Group scales and zeros: identical binary16 values / integers, row by row,
    up to the row's first divergence.  The GPU carries fp32 working weights,
    so a working value x differs from the oracle's by a rounding error; call
    its size, in grid steps of the value's group, eta.  A rounding decision
    can then come out differently only when the float64 quantity sits within
    that error of the decision boundary, and the three boundaries follow from
    the one budget:
      - code: the quotient x/s lies within ETA of the half-integer between
        the two codes (x moves by eta steps, x/s by eta);
      - zero: -lo/s lies within 3 ETA of k + 1/2 (lo moves by eta steps, and s
        by the relative amount below, which moves -lo/s by at most 2 eta more
        since |lo/s| <= maxq);
      - scale: the unrounded step (hi - lo)/maxq, or 2 max|v|/maxq, lies
        within 2 ETA / maxq (relative) of the midpoint between the two
        adjacent binary16 values (hi and lo each move by eta steps).
    ETA = 2e-4 steps is 13x the largest working-value error that fp32
    arithmetic of this kind (fp32 column loop, trailing update with products
    as exact as fp32) makes before a row's first divergence: 1.6e-5 steps,
    measured by emulating that arithmetic on the CPU for 8192-column rows of
    the 70B-shaped layer (4-bit g128; 3.5e-6 at 2-bit g32).
    After that point the row legitimately follows another greedy path (the
    error fed forward differs by one grid step), so later scale/zero
    differences in that row are counted, not failed, and bounded in number.
  * Codes: at most 0.5% of all codes differ.  Where a group's scale and zero
    agree, a differing code differs by exactly 1.  In a group whose parameters
    moved (only possible downstream of an admissible first divergence) codes
    are not comparable; there the dequantized values must agree to within two
    grid steps of the coarser grid (the working values differ by the one-step
    feedback difference fed forward from the divergence, and each side rounds
    by up to half a step), and such groups must stay under 1% of all groups.
  * Layer loss tr((W - What) H0 (W - What)^T): within 1e-3 relative.
"""
from __future__ import annotations

import numpy as np

ETA = 2e-4   # working-value error budget, in grid steps


def h_rel_error(H_gpu: np.ndarray, H_ref: np.ndarray) -> float:
    lo_g = np.tril(np.asarray(H_gpu, np.float64))
    lo_r = np.tril(np.asarray(H_ref, np.float64))
    return float(np.linalg.norm(lo_g - lo_r) / max(np.linalg.norm(lo_r), 1e-300))


def dequant(codes, scales, zeros, group_size):
    codes = np.asarray(codes, np.float64)
    d_in = codes.shape[1]
    G = d_in if group_size == -1 else group_size
    s = np.repeat(np.asarray(scales, np.float64), G, axis=1)[:, :d_in]
    z = np.repeat(np.asarray(zeros, np.float64), G, axis=1)[:, :d_in]
    return s * (codes - z)


def _scale_near_tie(sg, sr, raw, maxq):
    lo, hi = sorted((float(sg), float(sr)))
    nxt = float(np.nextafter(np.float16(lo), np.float16(np.inf)))
    return hi == nxt and abs(raw - 0.5 * (lo + nxt)) <= 2.0 * ETA / maxq * raw


def _zero_near_tie(zg, zr, raw):
    k = min(zg, zr)
    return abs(zg - zr) == 1 and abs(raw - (k + 0.5)) <= 3.0 * ETA


def compare_quant(gpu: dict, ref: dict, *, group_size: int, bits: int, W=None, H0=None,
                  max_code_frac: float = 0.005, loss_rtol: float = 1e-3,
                  max_row_frac: float = 0.05, max_param_frac: float = 0.01,
                  max_moved_steps: float = 2.0) -> dict:
    """Check GPU quantizer outputs against the oracle's; returns a report dict.

    gpu: codes, scales, zeros (numpy).  ref: the oracle's gptq() result.
    Raises AssertionError with the report when a bound is violated.
    """
    maxq = (1 << bits) - 1
    cg, cr = np.asarray(gpu["codes"]).astype(np.int64), np.asarray(ref["codes"]).astype(np.int64)
    sg, sr = np.asarray(gpu["scales"], np.float64), np.asarray(ref["scales"], np.float64)
    zg, zr = np.asarray(gpu["zeros"], np.float64), np.asarray(ref["zeros"], np.float64)
    d_out, d_in = cg.shape
    G = d_in if group_size == -1 else group_size
    rep = {"groups": int(sg.size)}
    pmis = (sg != sr) | (zg != zr)
    cmis = cg != cr
    rep["param_mismatch"] = int(pmis.sum())
    diff = np.abs(cg - cr)
    same = np.repeat(~pmis, G, axis=1)[:, :d_in]
    rep["code_diff_frac"] = float(cmis.mean()) if cmis.size else 0.0
    rep["code_max_diff"] = int(diff[same].max()) if same.any() else 0
    moved = ~same
    if moved.any():
        wg = dequant(cg, sg, zg, group_size)[moved]
        wr = dequant(cr, sr, zr, group_size)[moved]
        step = np.maximum(np.repeat(sg, G, axis=1)[:, :d_in], np.repeat(sr, G, axis=1)[:, :d_in])[moved]
        rep["moved_group_max_steps"] = float(np.max(np.abs(wg - wr) / step))
    else:
        rep["moved_group_max_steps"] = 0.0
    rep["codes_in_range"] = bool(cg.size == 0 or (cg.min() >= 0 and cg.max() <= maxq))
    rows = np.nonzero(pmis.any(axis=1) | cmis.any(axis=1))[0]
    rep["rows_diverged"] = int(rows.size)
    bad = []
    for r in rows:
        gcols = np.nonzero(pmis[r])[0] * G
        ccols = np.nonzero(cmis[r])[0]
        first_p = int(gcols.min()) if gcols.size else d_in
        first_c = int(ccols.min()) if ccols.size else d_in
        if first_p <= first_c:  # parameters differ first (at a group start)
            g = first_p // G
            if sg[r, g] != sr[r, g]:
                ok = _scale_near_tie(sg[r, g], sr[r, g], ref["raw_scales"][r, g], maxq)
            else:
                ok = _zero_near_tie(zg[r, g], zr[r, g], ref["raw_zeros"][r, g])
            what = ("param", g, float(sg[r, g]), float(sr[r, g]), float(zg[r, g]), float(zr[r, g]))
        else:
            j = first_c
            g = j // G
            k = min(cg[r, j], cr[r, j])
            boundary = (k - zr[r, g]) + 0.5
            rq = ref["raw_q"][r, j]
            ok = abs(cg[r, j] - cr[r, j]) == 1 and abs(rq - boundary) <= ETA
            what = ("code", j, int(cg[r, j]), int(cr[r, j]), float(rq))
        if not ok:
            bad.append((int(r),) + what)
    rep["first_divergence_inadmissible"] = bad[:10]
    if W is not None and H0 is not None:
        from oracle import layer_loss
        wh_g = dequant(gpu["codes"], gpu["scales"], gpu["zeros"], group_size)
        lg = layer_loss(W, wh_g, H0)
        lr = layer_loss(W, ref["What"], H0)
        rep["loss_gpu"], rep["loss_ref"] = lg, lr
        rep["loss_rel"] = abs(lg - lr) / max(abs(lr), 1e-300)
    problems = []
    if bad:
        problems.append("a row first diverges away from a rounding near-tie")
    if not rep["codes_in_range"]:
        problems.append("code out of range")
    if rep["code_max_diff"] > 1:
        problems.append("code differs by more than 1 under identical group parameters")
    # a moved group lies after the row's first (admissible) divergence: see
    # the module docstring for the two-step bound
    if rep["moved_group_max_steps"] > max_moved_steps:
        problems.append("dequantized value off by more than max_moved_steps in a moved group")
    if rep["param_mismatch"] > max_param_frac * rep["groups"]:
        problems.append("too many groups with moved parameters")
    if rep["code_diff_frac"] > max_code_frac:
        problems.append("too many differing codes")
    # each row takes d_in rounding decisions, each with a small chance of
    # sitting within the working-value error of a boundary, so the expected
    # share of rows that diverge grows with the row length: the bar is
    # max_row_frac at 4096 columns and scales linearly above that
    row_bar = max_row_frac * max(1.0, d_in / 4096.0)
    rep["row_bar"] = row_bar
    if d_out and rows.size > max(1, row_bar * d_out):
        problems.append("too many diverged rows")
    if "loss_rel" in rep and rep["loss_rel"] > loss_rtol:
        problems.append("layer loss outside tolerance")
    assert not problems, (problems, rep)
    return rep


def check_row_losses(gpu_loss, gpu: dict, ref: dict, rtol: float = 1e-4,
                     layer_rtol: float = 1e-3):
    """The damped loss sum_j delta_j^2 per row (the quantizer's loss_rows) against
    the oracle's.  A row whose codes and parameters all agree took the same
    greedy path, so its loss differs only by fp32 rounding of d_in squared
    terms (relative error far below rtol); a row that diverged (admissibly, at
    a near-tie) then follows another path and only enters the layer total,
    which stays within layer_rtol."""
    gl = np.asarray(gpu_loss, np.float64)
    rl = np.asarray(ref["loss_damped"], np.float64)
    same = ~((np.asarray(gpu["codes"]) != np.asarray(ref["codes"])).any(axis=1)
             | (np.asarray(gpu["scales"]) != np.asarray(ref["scales"])).any(axis=1)
             | (np.asarray(gpu["zeros"]) != np.asarray(ref["zeros"])).any(axis=1))
    np.testing.assert_allclose(gl[same], rl[same], rtol=rtol)
    assert abs(gl.sum() - rl.sum()) <= layer_rtol * abs(rl.sum())
    return int(same.sum())
