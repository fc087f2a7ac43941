"""Thin ctypes binding of libgptq_mi355x.so (C ABI in include/gptq.h).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch provides device memory (tensors, workspaces) and the stream.  The
functions keep the C names; tensors replace raw pointers, and outputs that the
caller does not pass in are allocated here with torch.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq_mi355x.so")

GPTQ_OK, GPTQ_EINVAL, GPTQ_EUNSUPPORTED, GPTQ_EHIP, GPTQ_ENOTSPD = range(5)
GPTQ_BF16, GPTQ_F32 = 0, 1

_lib = None


class GPTQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} (status {status})")
        self.status = status


class SyncTimeoutError(GPTQError):
    def __init__(self, where: str):
        RuntimeError.__init__(self, f"{where}: a bounded wait between workgroups expired "
                                    "(dev_status -1); the factorization did not complete")
        self.status = GPTQ_EHIP


def _raise_status(st: int, where: str):
    if st > 0:
        raise NotSPDError(st)
    if st < 0:
        raise SyncTimeoutError(where)


class NotSPDError(GPTQError):
    def __init__(self, pivot: int):
        RuntimeError.__init__(self, f"gptq_prepare_hinv: Hessian not positive definite "
                                    f"(pivot index {pivot - 1})")
        self.status = GPTQ_ENOTSPD
        self.pivot = pivot


def lib() -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m post_weight_quantization_syrk_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I, SZ, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
    sig = {
        "gptq_hessian_accumulate": (I, [P, I64, P, I, I64, I64, P, SZ, P]),
        "gptq_hessian_workspace": (SZ, [I64, I64, I]),
        "gptq_hessian_accumulate_noalloc": (I, [P, I64, P, I, I64, I64, P]),
        "gptq_noalloc_scratch_bytes": (SZ, []),
        "gptq_prepare_hinv": (I, [P, I64, D, P, P, P, P, SZ, P]),
        "gptq_prepare_workspace": (SZ, [I64]),
        "gptq_quantize_layer": (I, [P, I, I64, I64, P, P, I, I, I, I, P, P, P, P, P, SZ, P]),
        "gptq_quantize_workspace": (SZ, [I64, I64, I]),
        "gptq_pack": (I, [P, P, P, I64, I64, I, I, I, P, P, P, P]),
        "gptq2d_round": (I, [P, P, P, I64, P, P, SZ, P]),
        "gptq_w4a16_matmul": (I, [P, I64, I64, P, P, P, I64, I64, I, I, P, P]),
        "gptq_quantize_layers": (I, [P, P, I, I, I64, P, P, I, I, I, I, P, P, P, P, P, SZ, P]),
        "gptq_act_order": (I, [P, I, I64, I64, I64, P, P, P, SZ, P]),
        "gptq_act_order_workspace": (SZ, [I64, I64]),
        "gptq_prepare_hinv_perm": (I, [P, I64, D, P, P, P, P, P, SZ, P]),
        "gptq_quantize_layer_perm": (I, [P, I, I64, I64, P, P, P, I, I, I, I, I, P, P, P, P, P,
                                         P, SZ, P]),
        "gptq_quantize_perm_workspace": (SZ, [I64, I64, I]),
        "gptq2d_workspace": (SZ, [I64]),
        "gptq_strerror": (ctypes.c_char_p, [I]),
        "gptq_abi_version": (I, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().gptq_strerror(status).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != GPTQ_OK:
        raise GPTQError(status, where)


def _empty(stream, *args, **kw) -> torch.Tensor:
    """torch.empty, allocated on the stream the call will launch on: the
    caching allocator then hands the block out again only in that stream's
    order, so a buffer dropped when the call returns (its scratch) cannot be
    reused while the call's kernels still run on a stream other than the
    current one."""
    if stream is None:
        return torch.empty(*args, **kw)
    with torch.cuda.stream(stream):
        return torch.empty(*args, **kw)


def _workspace(nbytes: int, device, stream=None) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return _empty(stream, nbytes, dtype=torch.uint8, device=device)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GPTQ_BF16
    if t.dtype == torch.float32:
        return GPTQ_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


# --------------------------------------------------------------------------
def gptq_hessian_workspace(d: int, n_tokens: int, x_dtype: int) -> int:
    return int(lib().gptq_hessian_workspace(d, n_tokens, x_dtype))


def gptq_hessian_accumulate(H: torch.Tensor, X: torch.Tensor, ws: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """H (lower triangle) += 2 X^T X.  H [d, d] fp32; X [n, d] (row stride may exceed d)."""
    d = H.shape[0]
    if X.dim() != 2 or X.stride(1) != 1 or H.dtype != torch.float32 or not H.is_contiguous():
        raise ValueError("H must be contiguous fp32 [d, d]; X a row-major [n, >=d] matrix")
    if X.shape[1] < d:
        raise ValueError("X has fewer columns than d")
    xd = _dtype_code(X)
    n = X.shape[0]
    need = gptq_hessian_workspace(d, n, xd)
    if ws is None:
        ws = _workspace(need, H.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq_hessian_accumulate(_ptr(H), d, _ptr(X), xd, n, X.stride(0), _ptr(ws),
                                         nbytes, _stream(stream)), "gptq_hessian_accumulate")
    return H


def gptq_hessian_accumulate_noalloc(H: torch.Tensor, X: torch.Tensor, stream=None) -> torch.Tensor:
    """H (lower triangle) += 2 X^T X with the library's fixed per-GPU scratch: no
    device memory is allocated by this call (nor by the library)."""
    d = H.shape[0]
    if X.dim() != 2 or X.stride(1) != 1 or H.dtype != torch.float32 or not H.is_contiguous():
        raise ValueError("H must be contiguous fp32 [d, d]; X a row-major [n, >=d] matrix")
    if X.shape[1] < d:
        raise ValueError("X has fewer columns than d")
    _check(lib().gptq_hessian_accumulate_noalloc(_ptr(H), d, _ptr(X), _dtype_code(X), X.shape[0],
                                                 X.stride(0), _stream(stream)),
           "gptq_hessian_accumulate_noalloc")
    return H


def gptq_noalloc_scratch_bytes() -> int:
    return int(lib().gptq_noalloc_scratch_bytes())


def gptq_prepare_workspace(d: int) -> int:
    return int(lib().gptq_prepare_workspace(d))


def gptq_prepare_hinv(H: torch.Tensor, damp: float = 0.01, U: torch.Tensor | None = None,
                      dead: torch.Tensor | None = None, status: torch.Tensor | None = None,
                      ws: torch.Tensor | None = None, stream=None, check: bool = True):
    """Damp H in place and compute U (U^T U = H^-1).  Returns (U, dead, status).

    With check=True the stream is synchronised and a breakdown raises NotSPDError.
    """
    d = H.shape[0]
    dev = H.device
    if U is None:
        U = _empty(stream, (d, d), dtype=torch.float32, device=dev)
    if dead is None:
        dead = _empty(stream, d, dtype=torch.uint8, device=dev)
    if status is None:
        status = _empty(stream, 1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = _workspace(gptq_prepare_workspace(d), dev, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq_prepare_hinv(_ptr(H), d, float(damp), _ptr(U), _ptr(dead), _ptr(status),
                                   _ptr(ws), nbytes, _stream(stream)), "gptq_prepare_hinv")
    if check:
        (torch.cuda.current_stream() if stream is None else stream).synchronize()
        _raise_status(int(status.item()), "gptq_prepare_hinv")
    return U, dead, status


def gptq_quantize_workspace(d_out: int, d_in: int, block: int = 128) -> int:
    return int(lib().gptq_quantize_workspace(d_out, d_in, block))


def n_groups_for(d_in: int, group_size: int) -> int:
    return 1 if group_size == -1 else d_in // group_size


def gptq_quantize_layer(W: torch.Tensor, U: torch.Tensor, dead: torch.Tensor | None = None, *,
                        bits: int = 4, group_size: int = 128, sym: bool = False,
                        block: int = 128, codes=None, scales=None, zeros=None, loss_rows=None,
                        want_loss: bool = True, ws=None, stream=None):
    """Returns (codes uint8, scales fp32, zeros fp32, loss_rows fp32 or None)."""
    d_out, d_in = W.shape
    dev = W.device
    if not W.is_contiguous() or not U.is_contiguous():
        raise ValueError("W and U must be contiguous")
    ng = n_groups_for(d_in, group_size) if group_size > 0 or group_size == -1 else 1
    if codes is None:
        codes = _empty(stream, (d_out, d_in), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = _empty(stream, (d_out, max(ng, 1)), dtype=torch.float32, device=dev)
    if zeros is None:
        zeros = _empty(stream, (d_out, max(ng, 1)), dtype=torch.float32, device=dev)
    if loss_rows is None and want_loss:
        loss_rows = _empty(stream, d_out, dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(gptq_quantize_workspace(d_out, d_in, block), dev, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq_quantize_layer(_ptr(W), _dtype_code(W), d_out, d_in, _ptr(U), _ptr(dead),
                                     bits, group_size, int(bool(sym)), block, _ptr(codes),
                                     _ptr(scales), _ptr(zeros), _ptr(loss_rows), _ptr(ws),
                                     nbytes, _stream(stream)), "gptq_quantize_layer")
    return codes, scales, zeros, loss_rows


# -------------------------------------------------- layers sharing one Hessian
def gptq_quantize_layers(Ws: list, U: torch.Tensor, dead: torch.Tensor | None = None, *,
                         bits: int = 4, group_size: int = 128, sym: bool = False,
                         block: int = 128, want_loss: bool = True, ws=None, stream=None):
    """Quantize several matrices [d_out_i, d_in] that share U in one call.  Returns
    (codes, scales, zeros, loss_rows) stacked by rows in list order, and the list of
    per-matrix row slices."""
    if not Ws:
        raise ValueError("no matrices")
    d_in = Ws[0].shape[1]
    dt = _dtype_code(Ws[0])
    for w in Ws:
        if w.dim() != 2 or w.shape[1] != d_in or not w.is_contiguous() or _dtype_code(w) != dt:
            raise ValueError("matrices must be contiguous [d_out_i, d_in] of one dtype")
    dev = Ws[0].device
    rows = [int(w.shape[0]) for w in Ws]
    total = sum(rows)
    ng = n_groups_for(d_in, group_size) if group_size > 0 or group_size == -1 else 1
    codes = _empty(stream, (total, d_in), dtype=torch.uint8, device=dev)
    scales = _empty(stream, (total, max(ng, 1)), dtype=torch.float32, device=dev)
    zeros = _empty(stream, (total, max(ng, 1)), dtype=torch.float32, device=dev)
    loss_rows = _empty(stream, total, dtype=torch.float32, device=dev) if want_loss else None
    if ws is None:
        ws = _workspace(gptq_quantize_workspace(total, d_in, block), dev, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    ptrs = (ctypes.c_void_p * len(Ws))(*[w.data_ptr() for w in Ws])
    dl = (ctypes.c_int64 * len(Ws))(*rows)
    _check(lib().gptq_quantize_layers(ptrs, dl, len(Ws), dt, d_in, _ptr(U), _ptr(dead), bits,
                                      group_size, int(bool(sym)), block, _ptr(codes),
                                      _ptr(scales), _ptr(zeros), _ptr(loss_rows), _ptr(ws),
                                      nbytes, _stream(stream)), "gptq_quantize_layers")
    offs, slices = 0, []
    for r in rows:
        slices.append(slice(offs, offs + r))
        offs += r
    return codes, scales, zeros, loss_rows, slices


# -------------------------------------------------- activation ordering
def gptq_act_order_workspace(d: int, n_tokens: int) -> int:
    return int(lib().gptq_act_order_workspace(d, n_tokens))


def gptq_act_order(X: torch.Tensor, d: int | None = None, perm=None, act_sum=None, ws=None,
                   stream=None):
    """perm [d] int32: columns by ascending sum_t |X[t, c]|, ties by index.
    Returns (perm, act_sum float64 or None)."""
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a row-major [n, >=d] matrix")
    d = X.shape[1] if d is None else d
    n = X.shape[0]
    if perm is None:
        perm = _empty(stream, d, dtype=torch.int32, device=X.device)
    if ws is None:
        ws = _workspace(gptq_act_order_workspace(d, n), X.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq_act_order(_ptr(X), _dtype_code(X), n, X.stride(0), d, _ptr(perm),
                                _ptr(act_sum), _ptr(ws), nbytes, _stream(stream)),
           "gptq_act_order")
    return perm, act_sum


def gptq_prepare_hinv_perm(H: torch.Tensor, perm: torch.Tensor | None, damp: float = 0.01,
                           U=None, dead=None, status=None, ws=None, stream=None,
                           check: bool = True):
    """gptq_prepare_hinv for H[perm][:, perm].  Returns (U, dead, status)."""
    d = H.shape[0]
    dev = H.device
    if perm is not None and (perm.dtype != torch.int32 or perm.numel() != d):
        raise ValueError("perm must be an int32 tensor of d entries")
    if U is None:
        U = _empty(stream, (d, d), dtype=torch.float32, device=dev)
    if dead is None:
        dead = _empty(stream, d, dtype=torch.uint8, device=dev)
    if status is None:
        status = _empty(stream, 1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = _workspace(gptq_prepare_workspace(d), dev, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq_prepare_hinv_perm(_ptr(H), d, float(damp), _ptr(perm), _ptr(U), _ptr(dead),
                                        _ptr(status), _ptr(ws), nbytes, _stream(stream)),
           "gptq_prepare_hinv_perm")
    if check:
        (torch.cuda.current_stream() if stream is None else stream).synchronize()
        _raise_status(int(status.item()), "gptq_prepare_hinv_perm")
    return U, dead, status


def gptq_quantize_perm_workspace(d_out: int, d_in: int, block: int = 128) -> int:
    return int(lib().gptq_quantize_perm_workspace(d_out, d_in, block))


def gptq_quantize_layer_perm(W: torch.Tensor, U: torch.Tensor, dead: torch.Tensor | None,
                             perm: torch.Tensor | None, *, static_groups: bool = False,
                             bits: int = 4, group_size: int = 128, sym: bool = False,
                             block: int = 128, codes=None, scales=None, zeros=None, g_idx=None,
                             loss_rows=None, want_loss: bool = True, ws=None, stream=None):
    """Returns (codes uint8 in natural column order, scales, zeros, g_idx int32, loss_rows)."""
    d_out, d_in = W.shape
    dev = W.device
    if not W.is_contiguous() or not U.is_contiguous():
        raise ValueError("W and U must be contiguous")
    if perm is not None and (perm.dtype != torch.int32 or perm.numel() != d_in):
        raise ValueError("perm must be an int32 tensor of d_in entries")
    ng = n_groups_for(d_in, group_size) if group_size > 0 or group_size == -1 else 1
    if codes is None:
        codes = _empty(stream, (d_out, d_in), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = _empty(stream, (d_out, max(ng, 1)), dtype=torch.float32, device=dev)
    if zeros is None:
        zeros = _empty(stream, (d_out, max(ng, 1)), dtype=torch.float32, device=dev)
    if g_idx is None:
        g_idx = _empty(stream, d_in, dtype=torch.int32, device=dev)
    if loss_rows is None and want_loss:
        loss_rows = _empty(stream, d_out, dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(gptq_quantize_perm_workspace(d_out, d_in, block), dev, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq_quantize_layer_perm(_ptr(W), _dtype_code(W), d_out, d_in, _ptr(U),
                                          _ptr(dead), _ptr(perm), int(bool(static_groups)), bits,
                                          group_size, int(bool(sym)), block, _ptr(codes),
                                          _ptr(scales), _ptr(zeros), _ptr(g_idx),
                                          _ptr(loss_rows), _ptr(ws), nbytes, _stream(stream)),
           "gptq_quantize_layer_perm")
    return codes, scales, zeros, g_idx, loss_rows


def gptq_pack(codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor | None, *,
              bits: int, group_size: int, sym: bool, qweight=None, scales_f16=None,
              zeros_f16=None, stream=None):
    """Returns (qweight uint32 as int32 tensor, scales_f16 bits, zeros_f16 bits or None)."""
    d_out, d_in = codes.shape
    dev = codes.device
    words = (d_in * bits + 31) // 32
    ng = n_groups_for(d_in, group_size)
    if qweight is None:
        qweight = _empty(stream, (d_out, words), dtype=torch.int32, device=dev)
    if scales_f16 is None:
        scales_f16 = _empty(stream, (d_out, ng), dtype=torch.int16, device=dev)
    if zeros_f16 is None and not sym:
        zeros_f16 = _empty(stream, (d_out, ng), dtype=torch.int16, device=dev)
    _check(lib().gptq_pack(_ptr(codes), _ptr(scales), _ptr(zeros), d_out, d_in, bits, group_size,
                           int(bool(sym)), _ptr(qweight), _ptr(scales_f16), _ptr(zeros_f16),
                           _stream(stream)), "gptq_pack")
    return qweight, scales_f16, zeros_f16


# --------------------------------------------------------------------------
def gptq2d_workspace(n: int) -> int:
    return int(lib().gptq2d_workspace(n))


def gptq2d_round(Y: torch.Tensor, left_basis: torch.Tensor, right_basis: torch.Tensor,
                 Z: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """Two-sided rounding of Y [n, n] float64 under upper-triangular bases; returns Z (float64
    integers).  Only the bases' upper triangles are read."""
    n = Y.shape[0]
    for name, t in (("Y", Y), ("left_basis", left_basis), ("right_basis", right_basis)):
        if t.shape != (n, n) or t.dtype != torch.float64 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float64 [n, n] tensor")
    if Z is None:
        Z = _empty(stream, (n, n), dtype=torch.float64, device=Y.device)
    if ws is None:
        ws = _workspace(gptq2d_workspace(n), Y.device, stream)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq2d_round(_ptr(Y), _ptr(left_basis), _ptr(right_basis), n, _ptr(Z), _ptr(ws),
                              nbytes, _stream(stream)), "gptq2d_round")
    return Z


# --------------------------------------------------------------------------
def gptq_w4a16_matmul(X: torch.Tensor, qweight: torch.Tensor, scales_f16: torch.Tensor,
                      zeros_f16: torch.Tensor | None, *, group_size: int, sym: bool,
                      Y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y [m, d_out] fp32 = X [m, d_in] bf16 times the dequantized 4-bit weights (gptq_pack's
    qweight, scales_f16, zeros_f16) transposed."""
    if X.dtype != torch.bfloat16 or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a row-major bf16 [m, d_in] matrix")
    m, d_in = X.shape
    d_out = qweight.shape[0]
    if Y is None:
        Y = _empty(stream, (m, d_out), dtype=torch.float32, device=X.device)
    _check(lib().gptq_w4a16_matmul(_ptr(X), m, X.stride(0), _ptr(qweight), _ptr(scales_f16),
                                   _ptr(zeros_f16), d_out, d_in, group_size, int(bool(sym)),
                                   _ptr(Y), _stream(stream)), "gptq_w4a16_matmul")
    return Y
