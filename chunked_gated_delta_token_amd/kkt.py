"""Python binding of the C ABI in ``include/kkt_solve.h``.

Argument marshalling only: torch provides device memory and the current
stream, every step of the computation runs in the HIP library.  There is no
fallback: without ``libkkt_solve.so`` (or off gfx950) the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # imported before the library so both share torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkkt_solve.so")

KKT_DTYPE_F32, KKT_DTYPE_BF16, KKT_DTYPE_F16 = 0, 1, 2
KKT_OK, KKT_ERR_INVALID_ARGUMENT, KKT_ERR_UNSUPPORTED, KKT_ERR_HIP = 0, 1, 2, 3

_TORCH_TO_KKT = {torch.float32: KKT_DTYPE_F32, torch.bfloat16: KKT_DTYPE_BF16, torch.float16: KKT_DTYPE_F16}

# Every function the header declares, with its ctypes signature.
SIGNATURES = {
    "kkt_solve": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]),
    "kkt_last_error": (ctypes.c_char_p, []),
    "kkt_version": (ctypes.c_int, []),
}

_lib = None


class KKTError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kkt_solve failed with status {status}: {message}")
        self.status = status


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load ``libkkt_solve.so``; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m chunked_gated_delta_token_amd.build` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def kkt_solve_raw(k_ptr, g_ptr, beta_ptr, cu_ptr, num_seqs, B, T, H, K, chunk_size, in_dtype, out_dtype,
                  out_ptr, stream_ptr) -> int:
    """Direct call of the C entry point with raw integers / pointers; returns the status."""
    lib = load_library()
    return lib.kkt_solve(k_ptr, g_ptr, beta_ptr, cu_ptr, num_seqs, B, T, H, K, chunk_size, in_dtype,
                         out_dtype, out_ptr, stream_ptr)


def last_error() -> str:
    return load_library().kkt_last_error().decode()


def version() -> int:
    return int(load_library().kkt_version())


def kkt_solve(k: torch.Tensor, g: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
              output_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Rows of (I + A)^{-1} per 64-token chunk, shape [B, T, H, 64].

    Mirrors the fused API of MindSpeed-Ops PR #135 (user-facing-change
    section): ``k`` [B,T,H,K] (bf16 / fp16 / fp32), ``g`` and ``beta``
    [B,T,H] fp32 or None, ``cu_seqlens`` int32 [N+1] or None (then B == 1),
    ``chunk_size`` must be 64 (ValueError otherwise), ``output_dtype``
    defaults to k's dtype.  ``out`` may be given (contiguous, [B,T,H,64]);
    otherwise it is allocated uninitialised, since the kernel writes every
    element.
    """
    if chunk_size != 64:
        raise ValueError("chunk_size must be 64")
    if k.dim() != 4:
        raise ValueError("k must be [B, T, H, K]")
    if k.dtype not in _TORCH_TO_KKT:
        raise TypeError(f"unsupported k dtype {k.dtype}")
    if not k.is_cuda:
        raise ValueError("k must be a device tensor")
    B, T, H, K = k.shape
    k = k.contiguous()
    for name, t in (("g", g), ("beta", beta)):
        if t is not None:
            if t.shape != (B, T, H) or t.dtype != torch.float32 or t.device != k.device:
                raise ValueError(f"{name} must be float32 [B,T,H] on k's device")
    g = None if g is None else g.contiguous()
    beta = None if beta is None else beta.contiguous()
    num_seqs = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != k.device:
            raise ValueError("cu_seqlens must be int32 [N+1] on k's device")
        cu_seqlens = cu_seqlens.contiguous()
        num_seqs = cu_seqlens.numel() - 1
    odt = k.dtype if output_dtype is None else output_dtype
    if odt not in _TORCH_TO_KKT:
        raise TypeError(f"unsupported output dtype {odt}")
    if out is None:
        out = torch.empty((B, T, H, 64), dtype=odt, device=k.device)
    elif out.shape != (B, T, H, 64) or out.dtype != odt or not out.is_contiguous() or out.device != k.device:
        raise ValueError("out must be contiguous [B,T,H,64] of the output dtype on k's device")
    s = stream if stream is not None else torch.cuda.current_stream(k.device)
    with torch.cuda.device(k.device):
        st = kkt_solve_raw(_ptr(k), _ptr(g), _ptr(beta), _ptr(cu_seqlens), num_seqs, B, T, H, K, chunk_size,
                           _TORCH_TO_KKT[k.dtype], _TORCH_TO_KKT[odt], _ptr(out), ctypes.c_void_p(s.cuda_stream))
    if st != KKT_OK:
        raise KKTError(st, last_error())
    return out


def chunk_gated_delta_rule_fwd_kkt_solve(k, g=None, beta=None, cu_seqlens=None, chunk_size=64,
                                         output_dtype=None):
    """The pages' name for the fused op (same semantics as ``kkt_solve``)."""
    return kkt_solve(k, g, beta, cu_seqlens, chunk_size, output_dtype)
