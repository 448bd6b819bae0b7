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
KKT_OPTION_SPLIT_MAX_TILES, KKT_OPTION_VALIDATE_CU_SEQLENS = 0, 1

_TORCH_TO_KKT = {torch.float32: KKT_DTYPE_F32, torch.bfloat16: KKT_DTYPE_BF16, torch.float16: KKT_DTYPE_F16}

# Every function the header declares, with its ctypes signature.
SIGNATURES = {
    "kkt_solve": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]),
    "kkt_solve_gate_cumsum": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "kkt_scaled_dot": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]),
    "kkt_solve_tril": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "kkt_set_option": (ctypes.c_int, [ctypes.c_int, ctypes.c_int64]),
    "kkt_get_option": (ctypes.c_int64, [ctypes.c_int]),
    "kkt_last_error": (ctypes.c_char_p, []),
    "kkt_version": (ctypes.c_int, []),
}

_lib = None


class KKTError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kkt_solve failed with status {status}: {message}")
        self.status = status


class KKTInvalidArgument(KKTError, ValueError):
    """KKT_ERR_INVALID_ARGUMENT: a pointer, size or dtype the call cannot take."""


class KKTUnsupported(KKTError, NotImplementedError):
    """KKT_ERR_UNSUPPORTED: a valid request this build does not serve (chunk
    size, head dimension, a device other than gfx950)."""


def _error(status: int) -> KKTError:
    """The exception for a non-OK status, with the library's message."""
    cls = {KKT_ERR_INVALID_ARGUMENT: KKTInvalidArgument, KKT_ERR_UNSUPPORTED: KKTUnsupported}.get(status, KKTError)
    return cls(status, last_error())


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


def set_option(option: int, value: int) -> None:
    """Process-wide library option (KKT_OPTION_SPLIT_MAX_TILES,
    KKT_OPTION_VALIDATE_CU_SEQLENS); raises on an invalid option or value."""
    st = load_library().kkt_set_option(option, int(value))
    if st != KKT_OK:
        raise _error(st)


def get_option(option: int) -> int:
    return int(load_library().kkt_get_option(option))


class option:
    """Context manager that sets an option and restores its previous value."""

    def __init__(self, opt: int, value: int):
        self.opt, self.value, self.old = opt, value, None

    def __enter__(self):
        self.old = get_option(self.opt)
        set_option(self.opt, self.value)
        return self

    def __exit__(self, *exc):
        set_option(self.opt, self.old)
        return False


def last_error() -> str:
    return load_library().kkt_last_error().decode()


def version() -> int:
    return int(load_library().kkt_version())


def _check_k(k):
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("k must be [B, T, H, K]")
    if not k.is_cuda:
        raise ValueError("k must be a device tensor")


def _k_inputs(k, g, beta, cu_seqlens, chunk_size, chunk_sizes=(64,)):
    """Shared checks of the entry points that take k; returns contiguous
    tensors and the number of sequences."""
    if chunk_size not in chunk_sizes:
        raise ValueError(f"chunk_size must be {' or '.join(str(c) for c in chunk_sizes)}")
    if k.dim() != 4:
        raise ValueError("k must be [B, T, H, K]")
    if k.dtype not in _TORCH_TO_KKT:
        raise TypeError(f"unsupported k dtype {k.dtype}")
    if not k.is_cuda:
        raise ValueError("k must be a device tensor")
    B, T, H, _ = k.shape
    for name, t in (("g", g), ("beta", beta)):
        if t is not None:
            if t.shape != (B, T, H) or t.dtype != torch.float32 or t.device != k.device:
                raise ValueError(f"{name} must be float32 [B,T,H] on k's device")
    g = None if g is None else g.contiguous()
    beta = None if beta is None else beta.contiguous()
    cu_seqlens, num_seqs = _cu_input(cu_seqlens, k.device)
    return k.contiguous(), g, beta, cu_seqlens, num_seqs


def _cu_input(cu_seqlens, device):
    if cu_seqlens is None:
        return None, 0
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != device:
        raise ValueError("cu_seqlens must be int32 [N+1] on the input's device")
    return cu_seqlens.contiguous(), cu_seqlens.numel() - 1


def _out_tensor(out, shape, dtype, device):
    if out is None:
        # uninitialised: the kernels write every element
        return torch.empty(shape, dtype=dtype, device=device)
    if out.shape != shape or out.dtype != dtype or not out.is_contiguous() or out.device != device:
        raise ValueError(f"out must be contiguous {list(shape)} of dtype {dtype} on the input's device")
    return out


class _OnStream:
    """Runs a call's copies, allocations and launch on the launch stream.

    With no stream given that is the current stream, and nothing more is
    needed.  With another stream, that stream first waits for the current
    one (the caller produced the inputs there), the contiguous copies and
    the outputs are made under it (so the caching allocator ties them to it),
    and on exit every caller tensor the launch touches is recorded on it, so
    its memory is not handed to new work before the launch is done with it.
    """

    def __init__(self, stream, device):
        self.device = device
        self.cur = torch.cuda.current_stream(device)
        self.stream = stream if stream is not None else self.cur
        self.side = self.stream != self.cur
        self.keep = []
        self._ctx = None

    def __enter__(self):
        if self.side:
            self.stream.wait_stream(self.cur)
        self._ctx = torch.cuda.stream(self.stream)
        self._ctx.__enter__()
        return self

    def uses(self, *tensors):
        """Caller tensors the launch reads or writes (None entries ignored)."""
        self.keep.extend(t for t in tensors if t is not None)

    def ptr(self):
        return ctypes.c_void_p(self.stream.cuda_stream)

    def __exit__(self, *exc):
        self._ctx.__exit__(*exc)
        if self.side:
            for t in self.keep:
                t.record_stream(self.stream)
        return False


def kkt_solve(k: torch.Tensor, g: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
              output_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Rows of (I + A)^{-1} per chunk, shape [B, T, H, chunk_size].

    Mirrors the fused API of MindSpeed-Ops PR #135 (user-facing-change
    section): ``k`` [B,T,H,K] (bf16 / fp16 / fp32), ``g`` and ``beta``
    [B,T,H] fp32 or None, ``cu_seqlens`` int32 [N+1] or None (then B == 1),
    ``output_dtype`` defaults to k's dtype.  ``chunk_size`` is 64, the API's
    value, or 128 (the chunk size of the GDR case page's tiling); anything
    else raises ValueError.  ``out`` may be given (contiguous,
    [B,T,H,chunk_size]); otherwise it is allocated uninitialised, since the
    kernel writes every element.
    """
    _check_k(k)
    odt = k.dtype if output_dtype is None else output_dtype
    if odt not in _TORCH_TO_KKT:
        raise TypeError(f"unsupported output dtype {odt}")
    with torch.cuda.device(k.device), _OnStream(stream, k.device) as on:
        on.uses(k, g, beta, cu_seqlens, out)
        k, g, beta, cu_seqlens, num_seqs = _k_inputs(k, g, beta, cu_seqlens, chunk_size, (64, 128))
        B, T, H, K = k.shape
        out = _out_tensor(out, (B, T, H, chunk_size), odt, k.device)
        st = kkt_solve_raw(_ptr(k), _ptr(g), _ptr(beta), _ptr(cu_seqlens), num_seqs, B, T, H, K, chunk_size,
                           _TORCH_TO_KKT[k.dtype], _TORCH_TO_KKT[odt], _ptr(out), on.ptr())
    if st != KKT_OK:
        raise _error(st)
    return out


def kkt_solve_gate_cumsum(k: torch.Tensor, g_decay: torch.Tensor, beta: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                          output_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                          g_out: Optional[torch.Tensor] = None, return_gate: bool = False,
                          stream: Optional[torch.cuda.Stream] = None):
    """``kkt_solve`` fed with the per-token log-decay ``g_decay`` [B,T,H]
    fp32: the kernel sums it within every chunk (the gate ``kkt_solve``
    takes) before using it.  With ``return_gate`` (or a given ``g_out``) the
    summed gate is written too and ``(out, g)`` is returned; ``g_out`` may be
    ``g_decay`` itself (in-place sum).  ``chunk_size`` 64 or 128, as for
    ``kkt_solve``."""
    if g_decay is None:
        raise ValueError("g_decay is required (use kkt_solve without a gate)")
    _check_k(k)
    odt = k.dtype if output_dtype is None else output_dtype
    if odt not in _TORCH_TO_KKT:
        raise TypeError(f"unsupported output dtype {odt}")
    if g_out is not None and not (g_out.is_contiguous() and g_out.dtype == torch.float32
                                  and g_out.shape == k.shape[:3] and g_out.device == k.device):
        raise ValueError(f"g_out must be contiguous {list(k.shape[:3])} of dtype torch.float32 on k's device")
    with torch.cuda.device(k.device), _OnStream(stream, k.device) as on:
        on.uses(k, g_decay, beta, cu_seqlens, out, g_out)
        k, g_decay, beta, cu_seqlens, num_seqs = _k_inputs(k, g_decay, beta, cu_seqlens, chunk_size, (64, 128))
        B, T, H, K = k.shape
        out = _out_tensor(out, (B, T, H, chunk_size), odt, k.device)
        if g_out is None and return_gate:
            g_out = torch.empty((B, T, H), dtype=torch.float32, device=k.device)
        st = load_library().kkt_solve_gate_cumsum(_ptr(k), _ptr(g_decay), _ptr(beta), _ptr(cu_seqlens), num_seqs,
                                                  B, T, H, K, chunk_size, _TORCH_TO_KKT[k.dtype], _TORCH_TO_KKT[odt],
                                                  _ptr(out), _ptr(g_out), on.ptr())
    if st != KKT_OK:
        raise _error(st)
    return (out, g_out) if g_out is not None else out


def kkt_scaled_dot(k: torch.Tensor, g: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                   out: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The first step of the unfused chain alone: the strictly lower A of
    every 64-token chunk, fp32 [B, T, H, 64], zeros on and above the diagonal
    (MindSpeed-Ops PR #135, PR description: chunk_scaled_dot_kkt_fwd).
    Arguments as for ``kkt_solve``."""
    _check_k(k)
    with torch.cuda.device(k.device), _OnStream(stream, k.device) as on:
        on.uses(k, g, beta, cu_seqlens, out)
        k, g, beta, cu_seqlens, num_seqs = _k_inputs(k, g, beta, cu_seqlens, chunk_size)
        B, T, H, K = k.shape
        out = _out_tensor(out, (B, T, H, 64), torch.float32, k.device)
        st = load_library().kkt_scaled_dot(_ptr(k), _ptr(g), _ptr(beta), _ptr(cu_seqlens), num_seqs, B, T, H, K,
                                           chunk_size, _TORCH_TO_KKT[k.dtype], _ptr(out), on.ptr())
    if st != KKT_OK:
        raise _error(st)
    return out


def kkt_solve_tril(A: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                   output_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The second step alone: rows of (I + strict_lower(A))^{-1} per 64-token
    chunk (MindSpeed-Ops PR #135, PR description: solve_tril).  ``A`` is fp32
    [B, T, H, 64]; only its strictly lower entries are read.  ``output_dtype``
    defaults to fp32."""
    if chunk_size != 64:
        raise ValueError("chunk_size must be 64")
    if A.dim() != 4 or A.shape[3] != 64 or A.dtype != torch.float32 or not A.is_cuda:
        raise ValueError("A must be a float32 device tensor [B, T, H, 64]")
    odt = torch.float32 if output_dtype is None else output_dtype
    if odt not in _TORCH_TO_KKT:
        raise TypeError(f"unsupported output dtype {odt}")
    with torch.cuda.device(A.device), _OnStream(stream, A.device) as on:
        on.uses(A, cu_seqlens, out)
        A = A.contiguous()
        B, T, H, _ = A.shape
        cu_seqlens, num_seqs = _cu_input(cu_seqlens, A.device)
        out = _out_tensor(out, (B, T, H, 64), odt, A.device)
        st = load_library().kkt_solve_tril(_ptr(A), _ptr(cu_seqlens), num_seqs, B, T, H, chunk_size,
                                           _TORCH_TO_KKT[odt], _ptr(out), on.ptr())
    if st != KKT_OK:
        raise _error(st)
    return out


def chunk_gated_delta_rule_fwd_kkt_solve(k, g=None, beta=None, cu_seqlens=None, chunk_size=64,
                                         output_dtype=None):
    """The pages' name for the fused op (same semantics as ``kkt_solve``)."""
    return kkt_solve(k, g, beta, cu_seqlens, chunk_size, output_dtype)


def chunk_scaled_dot_kkt_fwd(k, beta=None, g=None, cu_seqlens=None, chunk_size=64):
    """The pages' name for the first step of the unfused chain (same
    semantics as ``kkt_scaled_dot``; fp32 output)."""
    return kkt_scaled_dot(k, g, beta, cu_seqlens, chunk_size)


def solve_tril(A, cu_seqlens=None, output_dtype=None):
    """The pages' name for the second step (same semantics as ``kkt_solve_tril``)."""
    return kkt_solve_tril(A, cu_seqlens, 64, output_dtype)
