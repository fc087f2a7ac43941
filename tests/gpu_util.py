"""Device-side helpers shared by the GPU tests (no step of the method here)."""
from __future__ import annotations

import numpy as np
import torch

from post_weight_quantization_syrk_amd import gptq

DEV = "cuda:0"


def dev_bf16(bits_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(DEV).view(
        torch.bfloat16)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def gpu_quant(W_dev, U, dead, bits, g, sym) -> dict:
    codes, scales, zeros, loss = gptq.gptq_quantize_layer(W_dev, U, dead, bits=bits,
                                                          group_size=g, sym=sym)
    torch.cuda.synchronize()
    return dict(codes=codes.cpu().numpy(), scales=scales.cpu().numpy(),
                zeros=zeros.cpu().numpy(), loss=loss.cpu().numpy())


def cond_estimate(Hd, U, iters=25):
    """kappa_2 of the damped H from power iterations on H and on H^-1 = U^T U."""
    rng = np.random.default_rng(0)
    v = rng.standard_normal(Hd.shape[0])
    for _ in range(iters):
        v = Hd @ v
        v /= np.linalg.norm(v)
    w = rng.standard_normal(Hd.shape[0])
    for _ in range(iters):
        w = U.T @ (U @ w)
        w /= np.linalg.norm(w)
    return float((v @ (Hd @ v)) * (w @ (U.T @ (U @ w))))


def u_bar(d, kappa):
    """Bar on max |U_gpu - U_ref| / max |U_ref| for the same fp32 input H.
    Rounding errors of an fp32 factorization act like a relative perturbation
    of H of about sqrt(d) u (u = 2^-24, O(d)-long accumulations with
    independent roundings), and the upper factor of the inverse amplifies a
    relative perturbation of H by about sqrt(kappa(H)).  Measured on the
    70B-shaped Hessian (d = 8192, kappa 7.5e4): 0.0023 sqrt(d) u sqrt(kappa);
    the bar allows 0.01, and never less than the well-conditioned bar below."""
    r = np.sqrt(d) * 2.0 ** -24
    return max(spd_u_bar(d), 0.01 * r * np.sqrt(kappa))


def spd_u_bar(d):
    """Bar for well-conditioned test matrices: 0.25 sqrt(d) u with a floor of
    3e-7 (measured 0.03 to 0.13 sqrt(d) u from d = 64 to 4096, as LAPACK's
    fp32 factorization gives on the same matrices)."""
    return max(3e-7, 0.25 * np.sqrt(d) * 2.0 ** -24)


def oracle_h_chunks(xb: np.ndarray, chunk: int, dtype: str):
    """float64 chunks of stored X (bf16 bits or fp32), for the oracle's Hessian."""
    from post_weight_quantization_syrk_amd import synth
    for t0 in range(0, xb.shape[0], chunk):
        yield synth.as_f64(xb[t0:t0 + chunk], dtype)
