"""The triangular inverse's launch plan (csrc/inv_plan.h), host logic only.

The inverse L^{-1} is formed by recursive doubling: level s pairs the blocks
[a, b) and [b, e) (b = a + s, e = min(b + s, d)) and forms the pair's
lower-left block in two steps over 64 x 64 tiles,
    T[b:e, a:b] = L[b:e, a:b] M[a:b, a:b],   M[b:e, a:b] = -M[b:e, b:e] T[b:e, a:b],
with M's diagonal 64 x 64 blocks written by the factorization's panels.  Its
tiles run in the factorization's panel and band launches when their operands
are already complete, and in rounds after the chain otherwise.  This test
builds the planner for the host with g++, replays the plan prepare_perm_launch
issues, and checks by brute force, from the two formulas above rather than
from the planner's own rules, that every tile runs exactly once and only after
everything it reads is final: L's columns (final once a launch starts past
them), M's diagonal blocks (written with those columns), the M blocks of
lower levels and the pair's T tiles (written by strictly earlier launches).
No GPU.  (Prepare step of "GPTQ：基于近似二阶信息的大模型权重量化", 阶段一.)"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_syrk_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_plan", "drive_plan.cpp")
NB = 64
SIZES = [1, 63, 64, 65, 127, 128, 130, 200, 256, 300, 512, 700, 1000, 1024, 1500, 2048, 3000,
         4096, 5000, 8192, 11008]


@pytest.fixture(scope="module")
def plans(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("needs g++")
    exe = str(tmp_path_factory.mktemp("plan") / "drive_plan")
    r = subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", f"-I{CSRC}", DRIVER, "-o",
                        exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe, *map(str, SIZES)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
    out = {}
    for line in r.stdout.split("\n"):
        if not line.strip():
            continue
        tag, d, cfin, *items = line.split()
        out.setdefault(int(d), []).append(
            (tag, int(cfin), [tuple(int(v) for v in it.split(",")) for it in items]))
    return out


def _cdiv(a, b):
    return -(-a // b)


def _steps(d):
    """Every step (s, x) with its tile count."""
    s, out = NB, []
    while s < d:
        pairs, sb = _cdiv(d - s, 2 * s), s // NB
        out += [(s, 0, pairs * sb * sb), (s, 1, pairs * sb * sb)]
        s *= 2
    return out


def _tile(d, s, x, g):
    """Output block (row block, column block) of tile g of step (s, x), the
    pair's a, b, e, and the K range in 64-blocks."""
    sb = s // NB
    p, lt = divmod(g, sb * sb)
    major, minor = divmod(lt, sb)
    rt, ct = (sb - 1 - major, minor) if x else (minor, major)
    a = 2 * s * p
    b, e = a + s, min(a + 2 * s, d)
    return p, a, b, e, rt, ct


def _check_plan(d, launches):
    when = {}  # (s, x, g) -> launch index
    for li, (tag, cfin, items) in enumerate(launches):
        assert tag in "PBR"
        for s, x, g0, cnt in items:
            assert cnt > 0
            for g in range(g0, g0 + cnt):
                assert (s, x, g) not in when, f"tile {(s, x, g)} run twice"
                when[(s, x, g)] = li
    for s, x, n in _steps(d):
        for g in range(n):
            assert (s, x, g) in when, f"tile {(s, x, g)} never run"
    assert len(when) == sum(n for _, _, n in _steps(d))

    # who writes M's 64-block (R, C), R > C: the X tile of the level whose pair
    # has R in [b, e) and C in [a, b)
    def m_block_launch(R, C):
        s = NB
        while True:
            a = (C * NB) // (2 * s) * (2 * s)
            b, e = a + s, min(a + 2 * s, d)
            if b <= R * NB < e and a <= C * NB < b:
                sb = s // NB
                rt, ct = (R * NB - b) // NB, (C * NB - a) // NB
                g = (a // (2 * s)) * sb * sb + (sb - 1 - rt) * sb + ct
                return when[(s, 1, g)]
            s *= 2

    def m_ready(R, C, li, cfin):
        if R == C:  # diagonal block: written with L's columns
            return min((R + 1) * NB, d) <= cfin
        return m_block_launch(R, C) < li

    for (s, x, g), li in when.items():
        tag, cfin, _ = launches[li]
        p, a, b, e, rt, ct = _tile(d, s, x, g)
        i0 = b + NB * rt
        if i0 >= d:
            continue
        sb = s // NB
        if x == 0:
            # T[i0 block, a + 64 ct block] = sum_k L[i0, a + k] M[a + k, a + 64 ct], k >= 64 ct
            assert b <= cfin, f"T {(s, g)} reads L columns before {b}, final before {cfin}"
            for kk in range(ct, _cdiv(b - a, NB)):
                assert m_ready(a // NB + kk, a // NB + ct, li, cfin), (d, s, g, kk)
        else:
            # M[i0 block, a + 64 ct block] = -sum_k M[i0, b + k] T[b + k, a + 64 ct], k < 64 rt + 64
            for kk in range(_cdiv(min(NB * rt + NB, e - b), NB)):
                assert m_ready(i0 // NB, b // NB + kk, li, cfin), (d, s, g, kk)
                gt = p * sb * sb + ct * sb + kk  # the T tile (rt = kk, ct)
                assert when[(s, 0, gt)] < li, f"X {(s, g)} before its T tile {gt}"
    return sum(cnt for tag, _, items in launches if tag != "R" for *_, cnt in items)


@pytest.mark.parametrize("d", SIZES)
def test_inverse_plan_respects_every_dependency(plans, d):
    launches = plans[d]
    n_panels = _cdiv(d, 256) if d > 0 else 0
    assert [t for t, _, _ in launches[:2 * n_panels - 1]] == ["P", "B"] * (n_panels - 1) + ["P"]
    carried = _check_plan(d, launches)
    if d == 4096:
        # the bench shape: most tiles, and the last level's T step, ride with the factorization
        assert carried > len([1 for s, x, n in _steps(d) for _ in range(n)]) // 2
        last_t = [it for tag, _, items in launches if tag != "R" for it in items
                  if it[0] == 2048 and it[1] == 0]
        assert sum(it[3] for it in last_t) == 1024


def test_plan_checker_catches_a_misordered_plan(plans):
    """The checker itself: moving one X tile into the launch of its T tile fails it."""
    launches = [(t, c, list(items)) for t, c, items in plans[1024]]
    for li, (tag, cfin, items) in enumerate(launches):
        xs = [it for it in items if it[1] == 1 and it[0] == 64]
        if xs:
            s, x, g0, cnt = xs[0]
            tl = next(lj for lj, (_, _, its) in enumerate(launches)
                      for (s2, x2, h0, hc) in its if s2 == s and x2 == 0 and h0 <= g0 < h0 + hc)
            items.remove(xs[0])
            if cnt > 1:
                items.append((s, x, g0 + 1, cnt - 1))
            launches[tl][2].append((s, x, g0, 1))
            break
    with pytest.raises(AssertionError):
        _check_plan(1024, launches)
