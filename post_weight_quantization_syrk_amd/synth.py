"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module holds input generation only: random draws, the per-channel scale
patterns, outlier placement and the float32 -> bfloat16 encoding of the inputs.
It contains none of the quantization method's arithmetic, so both sides can use
it without sharing any step of the method.

Every tensor is drawn from ``numpy.random.default_rng([cfg, tensor, chunk])`` so
any chunk of tokens can be regenerated on its own.  The workloads stand in for
the pages' real calibration run (128 sequences x 2048 tokens of a 7B model's
activations, "GPTQ：基于近似二阶信息的大模型权重量化", 动手实践 and FAQ), which is not
available here.

Tensor ids: 0 = W, 1 = X tokens, 2 = per-channel scales of X, 3 = outlier
channels / entries, 4 = second weight matrix.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np


# --------------------------------------------------------------------------
# bfloat16 encoding (round to nearest even), used only to build inputs.
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg: int, tensor: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg, tensor, chunk])


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int              # seed namespace
    d_out: int
    d_in: int
    n_tokens: int
    bits: int
    group_size: int
    sym: bool
    x_dtype: str          # "f32" or "bf16"
    w_dtype: str          # "f32" or "bf16"
    w_sigma: float
    chunk_tokens: int     # tokens per seeded chunk
    scale_sigma: float = 1.0   # log-normal sigma of per-channel X scales (0 = none)
    n_outlier_channels: int = 0
    outlier_channel_factor: float = 1.0
    w_outlier_frac: float = 0.0
    w_outlier_factor: float = 1.0
    relu: bool = False
    block: int = 128
    damp: float = 0.01


# Single layer 256x256, fp32, 2048 tokens, 4 outlier input channels x20;
# 4-bit asymmetric, g=128.
SMALL = Workload("layer256_f32_2048tok_4bit_g128", cfg=1, d_out=256, d_in=256,
                 n_tokens=2048, bits=4, group_size=128, sym=False,
                 x_dtype="f32", w_dtype="f32", w_sigma=0.02, chunk_tokens=2048,
                 scale_sigma=0.0, n_outlier_channels=4, outlier_channel_factor=20.0)

# Llama-7B-shaped attention projection: W 4096x4096 bf16 with 0.1% entries x10,
# X 262144x4096 bf16 (128 sequences x 2048 tokens) with log-normal(0,1)
# per-channel scales; 4-bit asymmetric, g=128.
ATTN7B = Workload("attn_proj_4096x4096_262144tok_4bit_g128", cfg=2, d_out=4096,
                  d_in=4096, n_tokens=262144, bits=4, group_size=128, sym=False,
                  x_dtype="bf16", w_dtype="bf16", w_sigma=0.02, chunk_tokens=32768,
                  scale_sigma=1.0, w_outlier_frac=0.001, w_outlier_factor=10.0)

# FFN pair (3-bit symmetric, g=64): gate/up 11008x4096 share one X; down
# 4096x11008 with a ReLU-like input (about half zeros).
FFN_GATE = Workload("ffn_gate_11008x4096_131072tok_3bit_sym_g64", cfg=3, d_out=11008,
                    d_in=4096, n_tokens=131072, bits=3, group_size=64, sym=True,
                    x_dtype="bf16", w_dtype="bf16", w_sigma=0.02, chunk_tokens=16384,
                    scale_sigma=1.0)
FFN_DOWN = Workload("ffn_down_4096x11008_131072tok_3bit_sym_g64", cfg=33, d_out=4096,
                    d_in=11008, n_tokens=131072, bits=3, group_size=64, sym=True,
                    x_dtype="bf16", w_dtype="bf16", w_sigma=0.02, chunk_tokens=16384,
                    scale_sigma=1.0, relu=True)

# 70B-shaped layers, one at a time: 8192x8192 and 28672x8192, X 65536x8192
# with log-normal(0,1.5) channel scales.  Quantizer swept by the caller.
L70B_SQ = Workload("l70b_8192x8192_65536tok", cfg=4, d_out=8192, d_in=8192,
                   n_tokens=65536, bits=4, group_size=128, sym=False, x_dtype="bf16",
                   w_dtype="bf16", w_sigma=0.015, chunk_tokens=8192, scale_sigma=1.5)
L70B_UP = Workload("l70b_28672x8192_65536tok", cfg=44, d_out=28672, d_in=8192,
                   n_tokens=65536, bits=4, group_size=128, sym=False, x_dtype="bf16",
                   w_dtype="bf16", w_sigma=0.015, chunk_tokens=8192, scale_sigma=1.5)

WORKLOADS = {w.name: w for w in (SMALL, ATTN7B, FFN_GATE, FFN_DOWN, L70B_SQ, L70B_UP)}


def scaled(wl: Workload, *, d_out: int | None = None, d_in: int | None = None,
           n_tokens: int | None = None, chunk_tokens: int | None = None,
           **kw) -> Workload:
    """Same recipe at a reduced size (for CPU-feasible parity cases)."""
    import dataclasses
    n = wl.n_tokens if n_tokens is None else n_tokens
    c = min(wl.chunk_tokens, n) if chunk_tokens is None else chunk_tokens
    return dataclasses.replace(
        wl, name=f"{wl.name}@{d_out or wl.d_out}x{d_in or wl.d_in}x{n}",
        d_out=d_out or wl.d_out, d_in=d_in or wl.d_in, n_tokens=n, chunk_tokens=c, **kw)


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------
def channel_scales(wl: Workload) -> np.ndarray:
    """Per-input-channel multipliers s_c (float32)."""
    s = np.ones(wl.d_in, dtype=np.float32)
    if wl.scale_sigma > 0:
        z = _rng(wl.cfg, 2).standard_normal(wl.d_in)
        s = np.exp(wl.scale_sigma * z).astype(np.float32)
    if wl.n_outlier_channels:
        idx = _rng(wl.cfg, 3).choice(wl.d_in, wl.n_outlier_channels, replace=False)
        s[idx] *= np.float32(wl.outlier_channel_factor)
    return s


def x_chunk_f32(wl: Workload, chunk: int, scales: np.ndarray | None = None) -> np.ndarray:
    """Tokens [chunk*chunk_tokens, ...) of X as float32 (before any bf16 rounding)."""
    t0 = chunk * wl.chunk_tokens
    rows = min(wl.chunk_tokens, wl.n_tokens - t0)
    if rows <= 0:
        raise IndexError("chunk out of range")
    s = channel_scales(wl) if scales is None else scales
    x = _rng(wl.cfg, 1, chunk).standard_normal((rows, wl.d_in), dtype=np.float32)
    if wl.relu:
        np.maximum(x, 0, out=x)
    x *= s[None, :]
    return x


def n_chunks(wl: Workload) -> int:
    return (wl.n_tokens + wl.chunk_tokens - 1) // wl.chunk_tokens


def x_chunk(wl: Workload, chunk: int, scales: np.ndarray | None = None) -> np.ndarray:
    """Chunk of X in its storage encoding: float32 array, or uint16 bf16 bits."""
    x = x_chunk_f32(wl, chunk, scales)
    if wl.x_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def x_full(wl: Workload, threads: int | None = None) -> np.ndarray:
    """All of X in storage encoding (row-major [n_tokens, d_in])."""
    s = channel_scales(wl)
    dt = np.uint16 if wl.x_dtype == "bf16" else np.float32
    out = np.empty((wl.n_tokens, wl.d_in), dtype=dt)
    nc = n_chunks(wl)

    def work(c):
        t0 = c * wl.chunk_tokens
        blk = x_chunk(wl, c, s)
        out[t0:t0 + blk.shape[0]] = blk

    threads = threads or min(8, os.cpu_count() or 1, nc)
    if threads > 1 and nc > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(nc)))
    else:
        for c in range(nc):
            work(c)
    return out


def w_matrix(wl: Workload, tensor: int = 0) -> np.ndarray:
    """Weight matrix in storage encoding (float32 array or uint16 bf16 bits)."""
    rng = _rng(wl.cfg, tensor)
    w = (rng.standard_normal((wl.d_out, wl.d_in), dtype=np.float32)
         * np.float32(wl.w_sigma))
    if wl.w_outlier_frac > 0:
        n = w.size
        k = int(n * wl.w_outlier_frac)
        idx = _rng(wl.cfg, 3, 1).choice(n, k, replace=False)
        w.reshape(-1)[idx] *= np.float32(wl.w_outlier_factor)
    if wl.w_dtype == "bf16":
        return f32_to_bf16_bits(w)
    return w


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of values stored as float32 or bf16 bits."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Two-sided rounding inputs: Y n x n ~ N(0,1), bases triu(I + 0.1 N(0,1)).
# --------------------------------------------------------------------------
def two_sided_inputs(n: int, cfg: int = 5):
    y = _rng(cfg, 0, n).standard_normal((n, n))
    rl = np.triu(np.eye(n) + 0.1 * _rng(cfg, 1, n).standard_normal((n, n)))
    rr = np.triu(np.eye(n) + 0.1 * _rng(cfg, 2, n).standard_normal((n, n)))
    # Positive diagonal: 1 + 0.1 N(0,1) is positive with overwhelming
    # probability; enforce it so the bases are always nonsingular.
    for r in (rl, rr):
        d = np.diag(r).copy()
        bad = d <= 0.05
        if bad.any():
            idx = np.where(bad)[0]
            r[idx, idx] = 1.0
    return y, rl, rr
