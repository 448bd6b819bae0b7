"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of ``oracle/kkt_oracle.c`` with one plausible mistake
(a dropped term, a wrong sign or index, a transposed operand, the sequence
boundary bug the pages describe), compiled into a temporary library.  The
test runs every pin on it and requires at least one to fail.  CPU only; the
real oracle source is never modified.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kkt_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("gate_sign", "double d = g[ti] - g[tj];", "double d = g[tj] - g[ti];"),
    ("beta_on_column", "(beta != NULL) ? beta[ti] : 1.0", "(beta != NULL) ? beta[tj] : 1.0"),
    ("dot_drops_first_term", "for (int64_t c = 0; c < K; ++c) {\n                dot",
     "for (int64_t c = 1; c < K; ++c) {\n                dot"),
    ("diagonal_in_A", "for (int64_t j = 0; j < i; ++j) {\n            const int64_t tj",
     "for (int64_t j = 0; j <= i; ++j) {\n            const int64_t tj"),
    ("minus_A", "((i == j) ? 1.0 : 0.0) + A[i * L + j]", "((i == j) ? 1.0 : 0.0) - A[i * L + j]"),
    ("transposed_output", "            row[j] = (j < L) ? X[i * L + j] : 0.0;\n        }\n    }\n    return KKT_ORACLE_OK;",
     "            row[j] = (j < L) ? X[j * L + i] : 0.0;\n        }\n    }\n    return KKT_ORACLE_OK;"),
    ("elimination_sign", "W[r * w + x] -= f * W[c * w + x];", "W[r * w + x] += f * W[c * w + x];"),
    ("clamp_bound_5", "static const double GATE_CLAMP = 50.0;", "static const double GATE_CLAMP = 5.0;"),
    ("no_clamp", "if (clamp_gate) {\n                    if (d > GATE_CLAMP)",
     "if (0) {\n                    if (d > GATE_CLAMP)"),
    ("gate_of_wrong_token", "double d = g[ti] - g[tj];", "double d = g[ti] - g[tj + (j > 0 ? -H : 0)];"),
    # chunk length taken from the full T instead of the sequence end
    ("sequence_end_uses_T", "out->len[n] = (eos - t0 < chunk_size) ? (eos - t0) : chunk_size;",
     "out->len[n] = (T - t0 < chunk_size) ? (T - t0) : chunk_size;"),
    # chunk starts snapped to the global 64-token grid instead of the sequence start
    ("chunks_ignore_sequence_start", "out->t0[n] = t0;", "out->t0[n] = t0 - bos % chunk_size;"),
    # the split steps: A written transposed; solve_tril reading A's upper part
    ("scaled_dot_transposed", "for (int64_t j = 0; j < chunk_size; ++j) row[j] = (j < L) ? A[i * L + j] : 0.0;",
     "for (int64_t j = 0; j < chunk_size; ++j) row[j] = (j < L) ? A[j * L + i] : 0.0;"),
    ("solve_tril_reads_upper", "M[i * L + j] = (i == j) ? 1.0 : ((j < i) ? arow[j] : 0.0);",
     "M[i * L + j] = (i == j) ? 1.0 : arow[j];"),
    ("key_of_previous_token", "const double* kj = k + tj * K;", "const double* kj = k + (tj >= H ? tj - H : tj) * K;"),
    # the gate from per-token decays: exclusive instead of inclusive sum; the
    # sum not restarted at chunk starts inside a sequence; head 0's decays for
    # every head
    ("cumsum_exclusive", "run += a[idx];\n                g_out[idx] = run;",
     "g_out[idx] = run;\n                run += a[idx];"),
    ("cumsum_restarts_per_sequence_only", "            double run = 0.0;\n            for (int64_t i = 0; i < ch.len[c]",
     "            double run = (c > 0 && ch.b[c - 1] == ch.b[c] && ch.len[c - 1] == chunk_size)"
     " ? g_out[(ch.b[c] * T + ch.t0[c] - 1) * H + h] : 0.0;\n"
     "            for (int64_t i = 0; i < ch.len[c]"),
    ("cumsum_head_zero", "                run += a[idx];", "                run += a[idx - h];"),
    # chunks of 128: the chunk length capped at 64 whatever chunk_size says
    ("chunk_len_capped_at_64", "out->len[n] = (eos - t0 < chunk_size) ? (eos - t0) : chunk_size;",
     "out->len[n] = (eos - t0 < chunk_size) ? (eos - t0) : (chunk_size > 64 ? 64 : chunk_size);"),
]


def _build(src_text, tmpdir, name):
    c = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-w", "-o", so, c, "-lm"],
                   check=True, capture_output=True)
    lib = ctypes.CDLL(so)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.kkt_oracle_solve.argtypes = [dp, dp, dp, ip, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, dp]
    lib.kkt_oracle_solve.restype = ctypes.c_int
    lib.kkt_oracle_scaled_dot.argtypes = lib.kkt_oracle_solve.argtypes
    lib.kkt_oracle_scaled_dot.restype = ctypes.c_int
    lib.kkt_oracle_solve_tril.argtypes = [dp, ip, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, dp]
    lib.kkt_oracle_solve_tril.restype = ctypes.c_int
    lib.kkt_oracle_chunk_cumsum.argtypes = [dp, ip, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, dp]
    lib.kkt_oracle_chunk_cumsum.restype = ctypes.c_int
    return lib


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(t))


def _split(lib):
    def scaled_dot(k, g=None, beta=None, cu=None, chunk_size=64):
        k = np.ascontiguousarray(k, dtype=np.float64)
        B, T, H, K = k.shape
        g = None if g is None else np.ascontiguousarray(g, dtype=np.float64)
        beta = None if beta is None else np.ascontiguousarray(beta, dtype=np.float64)
        cu = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
        out = np.empty((B, T, H, chunk_size))
        rc = lib.kkt_oracle_scaled_dot(_ptr(k, ctypes.c_double), _ptr(g, ctypes.c_double),
                                       _ptr(beta, ctypes.c_double), _ptr(cu, ctypes.c_int32),
                                       0 if cu is None else len(cu) - 1, B, T, H, K, chunk_size, 1,
                                       _ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError(rc)
        return out

    def solve_tril(A, cu=None, chunk_size=64):
        A = np.ascontiguousarray(A, dtype=np.float64)
        B, T, H, _ = A.shape
        cu = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
        out = np.empty_like(A)
        rc = lib.kkt_oracle_solve_tril(_ptr(A, ctypes.c_double), _ptr(cu, ctypes.c_int32),
                                       0 if cu is None else len(cu) - 1, B, T, H, chunk_size,
                                       _ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError(rc)
        return out
    return scaled_dot, solve_tril


def _cumsum(lib):
    def cumsum(a, cu=None, chunk_size=64):
        a = np.ascontiguousarray(a, dtype=np.float64)
        B, T, H = a.shape
        cu = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
        out = np.zeros_like(a)
        rc = lib.kkt_oracle_chunk_cumsum(_ptr(a, ctypes.c_double), _ptr(cu, ctypes.c_int32),
                                         0 if cu is None else len(cu) - 1, B, T, H, chunk_size,
                                         _ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError(rc)
        return out
    return cumsum


def _solver(lib):
    ptr = _ptr

    def solve(k, g=None, beta=None, cu=None, chunk_size=64, clamp_gate=True):
        k = np.ascontiguousarray(k, dtype=np.float64)
        B, T, H, K = k.shape
        g = None if g is None else np.ascontiguousarray(g, dtype=np.float64)
        beta = None if beta is None else np.ascontiguousarray(beta, dtype=np.float64)
        cu = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
        out = np.empty((B, T, H, chunk_size))
        rc = lib.kkt_oracle_solve(ptr(k, ctypes.c_double), ptr(g, ctypes.c_double), ptr(beta, ctypes.c_double),
                                  ptr(cu, ctypes.c_int32), 0 if cu is None else len(cu) - 1,
                                  B, T, H, K, chunk_size, int(clamp_gate), ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError(rc)
        return out
    return solve


@pytest.fixture(scope="module")
def tmpdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_unmutated_copy_passes(tmpdir):
    with open(SRC) as f:
        lib = _build(f.read(), tmpdir, "clean")
    solve = _solver(lib)
    for pin in oracle_pins.ALL_PINS:
        pin(solve)
    for pin in oracle_pins.SPLIT_PINS:
        pin(solve, *_split(lib))
    for pin in oracle_pins.CUMSUM_PINS:
        pin(solve, _cumsum(lib))
    for pin in oracle_pins.CHUNK128_PINS:
        pin(solve)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmpdir, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    lib = _build(text.replace(old, new), tmpdir, name)
    solve = _solver(lib)
    scaled_dot, solve_tril = _split(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(solve)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    for pin in oracle_pins.SPLIT_PINS:
        try:
            pin(solve, scaled_dot, solve_tril)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    cumsum = _cumsum(lib)
    for pin in oracle_pins.CUMSUM_PINS:
        try:
            pin(solve, cumsum)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    for pin in oracle_pins.CHUNK128_PINS:
        try:
            pin(solve)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
