"""Dequantized matrix product with the packed weights, float64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P1] "GPTQ：基于近似二阶信息的大模型权重量化", 阶段三 (the quantized weights are
used as integers plus per-group scale and zero at inference) and [P5]
"GPTQ/AWQ量化中Group Size的精确含义与计算" (存储代价: b-bit codes with a 16-bit
scale and a zero point per group of g input columns):

  W_hat[n][k] = s[n][k // g] * (q[n][k] - z[n][k // g]),   Y = X W_hat^T,

with q unpacked from the little-endian bit stream of each row (the packing
of gptq_pack), s and z the binary16 values stored beside them, z = (maxq +
1) / 2 for a symmetric quantizer (no zero is stored), g = d_in for one group
per row.
"""
from __future__ import annotations

import numpy as np

from .gptq_oracle import maxq_for
from .storage import unpack_rows


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequantize(qweight, scales_f16, zeros_f16, *, bits, group_size, sym, d_in) -> np.ndarray:
    """W_hat [d_out, d_in] in float64 from the packed artifact."""
    q = unpack_rows(np.asarray(qweight).view(np.uint32), bits, d_in).astype(np.float64)
    G = d_in if group_size in (-1, None) else int(group_size)
    g = np.arange(d_in) // G
    s = f16_bits_to_f64(scales_f16)
    if sym:
        z = np.full_like(s, float((maxq_for(bits) + 1) // 2))
    else:
        z = f16_bits_to_f64(zeros_f16)
    return s[:, g] * (q - z[:, g])


def dequant_matmul(X, qweight, scales_f16, zeros_f16, *, bits, group_size, sym) -> np.ndarray:
    """Y = X W_hat^T in float64 (X [m, d_in])."""
    X = np.asarray(X, dtype=np.float64)
    W = dequantize(qweight, scales_f16, zeros_f16, bits=bits, group_size=group_size, sym=sym,
                   d_in=X.shape[1])
    return X @ W.T
