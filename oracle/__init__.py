"""CPU fp64 oracle for the fused chunk-local KKT + triangular solve.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports or calls it, and it
imports nothing from the product path.

The arithmetic lives in ``kkt_oracle.c`` (plain fp64 loops: explicit A, then a
generic Gauss-Jordan inverse with partial pivoting per chunk).  This module
compiles it with gcc, marshals numpy arrays through ctypes, and defines the
expected value of a rounded output (round-to-nearest-even from the exact fp64
result straight to the output format).

Sources: MindSpeed-Ops pull request #135 "feat(triton): add
chunk_gated_delta_rule_fwd_kkt_solve" (PR description; user-facing-change
section with the signature; bot change summary).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kkt_oracle.c")
_LIB = os.path.join(_HERE, "libkkt_oracle.so")

_lib = None


def build(quiet: bool = True, out: str = None, src: str = None, sanitize: bool = False) -> str:
    """Compile ``kkt_oracle.c`` into ``libkkt_oracle.so`` (gcc, OpenMP, fp64).

    -O2 without fast-math: the compiler keeps the written order of every
    floating-point operation.  ``out`` / ``src`` build another path or source
    (the tests' planted-mistake copies); ``sanitize`` adds AddressSanitizer
    and UndefinedBehaviorSanitizer (aborting on the first report), for the
    tests that run the pins on such a build.
    """
    out = out or _LIB
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra"]
    if sanitize:
        cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    cmd += ["-o", out + ".tmp", src or _SRC, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    os.replace(out + ".tmp", out)
    if not quiet:
        print("built", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("KKT_ORACLE_LIB") or _LIB  # (another build of the same source, e.g. sanitized)
    if path == _LIB and not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.kkt_oracle_solve.argtypes = [dp, dp, dp, ip, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int, dp]
    lib.kkt_oracle_solve.restype = ctypes.c_int
    lib.kkt_oracle_scaled_dot.argtypes = lib.kkt_oracle_solve.argtypes
    lib.kkt_oracle_scaled_dot.restype = ctypes.c_int
    lib.kkt_oracle_solve_tril.argtypes = [dp, ip, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, dp]
    lib.kkt_oracle_solve_tril.restype = ctypes.c_int
    lib.kkt_oracle_chunk_cumsum.argtypes = [dp, ip, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, dp]
    lib.kkt_oracle_chunk_cumsum.restype = ctypes.c_int
    lib.kkt_oracle_num_threads.argtypes = []
    lib.kkt_oracle_num_threads.restype = ctypes.c_int
    lib.kkt_oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.kkt_oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def num_threads() -> int:
    """Threads the oracle's parallel loop uses (OpenMP default)."""
    return int(_load().kkt_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later parallel loops (timing only)."""
    _load().kkt_oracle_set_num_threads(int(n))


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _kkt_call(fn_name, k, g, beta, cu_seqlens, chunk_size, clamp_gate):
    lib = _load()
    k64 = np.ascontiguousarray(k, dtype=np.float64)
    if k64.ndim != 4:
        raise ValueError("k must be [B,T,H,K]")
    B, T, H, K = k64.shape
    g64 = None if g is None else np.ascontiguousarray(g, dtype=np.float64)
    b64 = None if beta is None else np.ascontiguousarray(beta, dtype=np.float64)
    for name, a in (("g", g64), ("beta", b64)):
        if a is not None and a.shape != (B, T, H):
            raise ValueError(f"{name} must be [B,T,H]={B, T, H}, got {a.shape}")
    cu, num_seqs = _cu(cu_seqlens)
    out = np.empty((B, T, H, chunk_size), dtype=np.float64)
    rc = getattr(lib, fn_name)(_ptr(k64, ctypes.c_double), _ptr(g64, ctypes.c_double),
                               _ptr(b64, ctypes.c_double), _ptr(cu, ctypes.c_int32), num_seqs,
                               B, T, H, K, chunk_size, 1 if clamp_gate else 0, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"{fn_name} failed with code {rc}")
    return out


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None, 0
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    return cu, cu.shape[0] - 1


def scaled_dot_ref(k, g=None, beta=None, cu_seqlens=None, chunk_size: int = 64,
                   clamp_gate: bool = True) -> np.ndarray:
    """The first step alone: per chunk the strictly lower A (fp64), row
    t0+i holding A[i][0..chunk_size-1], zeros on and above the diagonal."""
    return _kkt_call("kkt_oracle_scaled_dot", k, g, beta, cu_seqlens, chunk_size, clamp_gate)


def solve_tril_ref(A, cu_seqlens=None, chunk_size: int = 64) -> np.ndarray:
    """The second step alone: rows of (I + strict_lower(A_chunk))^{-1} per
    chunk; A's diagonal and upper entries are ignored."""
    lib = _load()
    a64 = np.ascontiguousarray(A, dtype=np.float64)
    if a64.ndim != 4 or a64.shape[3] != chunk_size:
        raise ValueError("A must be [B,T,H,chunk_size]")
    B, T, H, _ = a64.shape
    cu, num_seqs = _cu(cu_seqlens)
    out = np.empty_like(a64)
    rc = lib.kkt_oracle_solve_tril(_ptr(a64, ctypes.c_double), _ptr(cu, ctypes.c_int32), num_seqs,
                                   B, T, H, chunk_size, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"kkt_oracle_solve_tril failed with code {rc}")
    return out


def chunk_cumsum_ref(a, cu_seqlens=None, chunk_size: int = 64) -> np.ndarray:
    """Chunk-local inclusive cumulative sum of a per-token log-decay ``a``
    [B,T,H] (fp64), restarted at every chunk: the gate the op takes."""
    lib = _load()
    a64 = np.ascontiguousarray(a, dtype=np.float64)
    if a64.ndim != 3:
        raise ValueError("a must be [B,T,H]")
    B, T, H = a64.shape
    cu, num_seqs = _cu(cu_seqlens)
    out = np.zeros_like(a64)
    rc = lib.kkt_oracle_chunk_cumsum(_ptr(a64, ctypes.c_double), _ptr(cu, ctypes.c_int32), num_seqs,
                                     B, T, H, chunk_size, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"kkt_oracle_chunk_cumsum failed with code {rc}")
    return out


def kkt_solve_gate_cumsum_ref(k, a, beta=None, cu_seqlens=None, chunk_size: int = 64,
                              clamp_gate: bool = True):
    """The fused op fed with the per-token log-decay ``a`` instead of its
    chunk-local sum: returns (rows of (I + A)^{-1}, the summed gate g)."""
    g = chunk_cumsum_ref(a, cu_seqlens, chunk_size)
    return kkt_solve_ref(k, g, beta, cu_seqlens, chunk_size, clamp_gate), g


def kkt_solve_ref(k, g=None, beta=None, cu_seqlens=None, chunk_size: int = 64,
                  clamp_gate: bool = True) -> np.ndarray:
    """Exact (fp64) rows of (I + A)^{-1} per chunk, shape [B, T, H, chunk_size].

    ``k`` [B,T,H,K], ``g`` / ``beta`` [B,T,H] (or None), ``cu_seqlens`` int
    [N+1] (or None; then B must be 1 for varlen).  Any real dtype is accepted;
    values are widened to fp64 (exact for fp32, fp16 and bf16 values).
    ``clamp_gate`` clamps g_i - g_j to [-50, 50] before exp, as the pages do.
    """
    return _kkt_call("kkt_oracle_solve", k, g, beta, cu_seqlens, chunk_size, clamp_gate)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 with round-to-nearest-even, directly from
    fp64 (no intermediate fp32 rounding), returning the uint16 bit patterns.

    bfloat16 keeps 8 significant bits.  For |x| in [2^e, 2^(e+1)) the spacing
    of bf16 values is 2^(e-7); below the smallest normal (2^-126) it is
    2^-133.  Division and multiplication by powers of two are exact in fp64,
    and np.rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    safe = np.where(ax > 0, ax, 1.0)
    e = np.floor(np.log2(safe))
    # log2 may be off by one near powers of two: fix e so that 2^e <= |x| < 2^(e+1)
    e = np.where(np.exp2(e) > safe, e - 1, e)
    e = np.where(np.exp2(e + 1) <= safe, e + 1, e)
    quantum = np.exp2(np.maximum(e - 7, -133.0))
    r = np.rint(x / quantum) * quantum
    r = np.where(ax > 0, r, x)  # keeps +0.0 / -0.0
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)  # exact: every bf16 value is an fp32 value (or overflows to inf)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


def round_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 to IEEE binary16 with round-to-nearest-even (numpy converts
    float64 to float16 directly), returning the uint16 bit patterns."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)
