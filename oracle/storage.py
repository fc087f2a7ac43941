"""Storage accounting and the packed code layout (reference side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Storage arithmetic follows [P5] 存储代价: each group carries one 16-bit scale
and, when asymmetric, one zero point of the code width, so the overhead per
weight is (16 + zero_bits) / group_size; symmetric groups store no zero and
the numerator drops to 16.  group_size = -1 makes the whole row one group
([P5]: "整个行是一个 group").

Packed layout (a reading: the pages give bit counts, not a layout): the codes
of one row form a little-endian bit stream, code j occupying bits
[b*j, b*j + b), cut into 32-bit words; a row takes ceil(d_in*b/32) words.
At 3 bits, 32 codes fill 3 words and codes straddle word boundaries.
"""
from __future__ import annotations

from decimal import Decimal, ROUND_HALF_UP

import numpy as np


def bits_per_weight(bits: int, group_size: int, sym: bool = False, d_in: int | None = None,
                    scale_bits: int = 16, zero_bits: int | None = None) -> float:
    """b + (scale_bits + zero_bits)/G; zero_bits defaults to the code width."""
    if group_size == -1:
        if d_in is None:
            raise ValueError("group_size=-1 needs d_in")
        G = d_in
    else:
        G = group_size
    zb = bits if zero_bits is None else zero_bits
    meta = scale_bits + (0 if sym else zb)
    return bits + meta / G


def model_gigabytes(n_weights: float, bpw: float) -> float:
    """Decimal gigabytes for n_weights at bpw bits each ([P5]: N * bpw / 8)."""
    return n_weights * bpw / 8.0 / 1e9


def round_half_up(x: float, digits: int) -> str:
    """Decimal rounding as the page prints (4.3125 -> 4.313)."""
    q = Decimal(1).scaleb(-digits)
    return str(Decimal(repr(x)).quantize(q, rounding=ROUND_HALF_UP))


def words_per_row(d_in: int, bits: int) -> int:
    return (d_in * bits + 31) // 32


def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack uint8 codes [rows, d_in] into uint32 words [rows, words_per_row]."""
    codes = np.asarray(codes, dtype=np.uint64)
    rows, d_in = codes.shape
    if np.any(codes >> np.uint64(bits)):
        raise ValueError("code out of range")
    nw = words_per_row(d_in, bits)
    out = np.zeros((rows, nw), dtype=np.uint64)
    for j in range(d_in):
        bit = bits * j
        w, off = divmod(bit, 32)
        out[:, w] |= (codes[:, j] << np.uint64(off)) & np.uint64(0xFFFFFFFF)
        spill = off + bits - 32
        if spill > 0:
            out[:, w + 1] |= codes[:, j] >> np.uint64(bits - spill)
    return out.astype(np.uint32)


def unpack_rows(words: np.ndarray, bits: int, d_in: int) -> np.ndarray:
    """Inverse of pack_rows."""
    words = np.asarray(words, dtype=np.uint64)
    rows = words.shape[0]
    mask = np.uint64((1 << bits) - 1)
    out = np.zeros((rows, d_in), dtype=np.uint8)
    for j in range(d_in):
        bit = bits * j
        w, off = divmod(bit, 32)
        v = words[:, w] >> np.uint64(off)
        if off + bits > 32:
            v |= words[:, w + 1] << np.uint64(32 - off)
        out[:, j] = (v & mask).astype(np.uint8)
    return out


def fp16_bits(values: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns of values that are exactly representable."""
    v = np.asarray(values, dtype=np.float64)
    h = v.astype(np.float16)
    if not np.array_equal(h.astype(np.float64), v):
        raise ValueError("value not representable in binary16")
    return h.view(np.uint16)
