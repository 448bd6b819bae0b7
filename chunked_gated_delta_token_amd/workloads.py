"""Seeded synthetic inputs for the fused chunk-local KKT + triangular solve.

This module only draws inputs.  It holds none of the method's arithmetic
(no K K^T, no gate, no solve), so the oracle and the HIP path can both take
their inputs from it.

Recipe (the shapes are those of the performance and generalisation tables on
the MindSpeed-Ops PR #135 page; the value distributions are the usual ones
for Gated DeltaNet inputs):

  1. varlen only: sequence lengths, ``n_seqs - 1`` integers uniform in
     [len_lo, len_hi], the last one = T - sum, redrawn from the same
     generator until it also lies in [len_lo, len_hi];
  2. k ~ N(0, 1) of shape [B,T,H,K] in fp64, L2-normalised per (token, head)
     in fp64, then rounded (round-to-nearest-even) to the input dtype;
  3. u_beta ~ N(0, 1) of shape [B,T,H]; beta = sigmoid(u_beta), rounded to fp32;
  4. u_g ~ N(4, 1) of shape [B,T,H]; g = chunk-local cumulative sum of
     logsigmoid(u_g) = -log1p(exp(-u_g)), in fp64, restarting at every
     64-token chunk and at every sequence start, rounded to fp32.  The
     per-token decays logsigmoid(u_g), rounded to fp32, are kept as g_raw
     (the input of the entry point that sums them itself).

Draws happen in that order from ``numpy.random.default_rng(seed)`` (PCG64);
steps 3 and 4 are skipped when the workload has no beta / no gate.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

CHUNK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    K: int
    in_dtype: str          # "bf16" | "f16" | "f32"
    out_dtype: str         # "bf16" | "f16" | "f32"
    gate: bool
    beta: bool
    seed: int
    n_seqs: int = 0        # 0: fixed length; > 0: B == 1 and packed varlen
    len_lo: int = 200
    len_hi: int = 3000
    note: str = field(default="", compare=False)


# The five workloads.  Names say what they are.
WORKLOADS = {
    w.name: w for w in (
        Workload("T256_H8_bf16_f32", 1, 256, 8, 128, "bf16", "f32", True, True, seed=0,
                 note="4 full chunks per head; small case the oracle finishes at once"),
        Workload("T2000_H8_bf16_bf16", 1, 2000, 8, 128, "bf16", "bf16", True, True, seed=1,
                 note="31 full chunks + one 16-token chunk per head"),
        Workload("T8192_H8_bf16_f32", 1, 8192, 8, 128, "bf16", "f32", True, True, seed=2,
                 note="1024 chunk-head tiles, 2 KiB row stride"),
        Workload("B2_T16384_H32_bf16_bf16", 2, 16384, 32, 128, "bf16", "bf16", True, True, seed=3,
                 note="16384 chunk-head tiles, 8 KiB row stride"),
        Workload("varlen12_T16384_H7_f32_f32", 1, 16384, 7, 128, "f32", "f32", False, False, seed=4,
                 n_seqs=12, note="12 packed sequences, partial chunks inside, odd H, no gate/beta"),
    )
}

# The bench workload: (B,T,H,K) = (1,8192,8,128), bf16 keys, fp32 output.
BENCH_WORKLOAD = "T8192_H8_bf16_f32"


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 to bfloat16 (round-to-nearest-even, straight from fp64) and
    return uint16 bit patterns.  Used to cast generated keys."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 22
    for a in range(0, flat.size, step):
        out[a:a + step] = _f64_to_bf16_bits_block(flat[a:a + step])
    return out.reshape(x.shape)


def _f64_to_bf16_bits_block(x: np.ndarray) -> np.ndarray:
    """

    Fast path on the fp64 bit pattern: drop the low 45 of the 52 mantissa
    bits with round-half-even (a carry may bump the exponent), then re-bias
    the exponent.  Results outside bf16's normal range take a slow exact path.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint16) << np.uint16(15)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    lsb = (mag >> np.uint64(45)) & np.uint64(1)
    r = (mag + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)       # 11-bit exponent | 7-bit mantissa
    e = (r >> np.uint64(7)).astype(np.int64) - 1023 + 127
    out = sign | (np.clip(e, 0, 255).astype(np.uint16) << np.uint16(7)) | (r & np.uint64(0x7F)).astype(np.uint16)
    out = np.where(mag == 0, sign, out)
    slow = (mag != 0) & ((e < 1) | (e > 254))
    if np.any(slow):
        xs = x[slow]
        m_, e_ = np.frexp(xs)                  # xs = m_ * 2^e_, 0.5 <= |m_| < 1
        q = np.maximum(e_ - 8, -133)           # bf16 keeps 8 significant bits, quantum >= 2^-133
        rs = np.ldexp(np.rint(np.ldexp(xs, -q)), q)
        with np.errstate(over="ignore"):
            out[slow] = (rs.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass
class Inputs:
    """Host arrays for one call.  ``k_store`` is what goes to the device:
    uint16 bit patterns for bf16/f16, float32 for f32.  ``k64`` is the same
    values widened exactly to fp64 (filled lazily for large workloads)."""
    workload: Workload
    k_store: np.ndarray
    g: Optional[np.ndarray]          # float32 [B,T,H] or None
    beta: Optional[np.ndarray]       # float32 [B,T,H] or None
    cu_seqlens: Optional[np.ndarray]  # int32 [N+1] or None
    g_raw: Optional[np.ndarray] = None  # float32 [B,T,H]: the per-token log-decays g sums, or None

    def k64(self, sl=None) -> np.ndarray:
        src = self.k_store if sl is None else self.k_store[sl]
        dt = self.workload.in_dtype
        if dt == "bf16":
            return bf16_bits_to_f64(src)
        if dt == "f16":
            return src.view(np.float16).astype(np.float64)
        return src.astype(np.float64)


def draw_lengths(rng: np.random.Generator, T: int, n: int, lo: int, hi: int) -> np.ndarray:
    if n * lo > T or n * hi < T:
        raise ValueError("lengths cannot sum to T")
    while True:
        head = rng.integers(lo, hi + 1, size=n - 1)
        last = T - int(head.sum())
        if lo <= last <= hi:
            return np.concatenate([head, [last]]).astype(np.int64)


def chunk_local_cumsum(x: np.ndarray, seq_starts: np.ndarray, T: int, chunk: int = CHUNK) -> np.ndarray:
    """Cumulative sum along T (axis 1 of [B,T,H]) restarting at every chunk of
    ``chunk`` tokens, counted from each sequence start in ``seq_starts``
    (which includes T as its last entry)."""
    out = np.empty_like(x)
    for s in range(len(seq_starts) - 1):
        bos, eos = int(seq_starts[s]), int(seq_starts[s + 1])
        for t0 in range(bos, eos, chunk):
            t1 = min(t0 + chunk, eos)
            out[:, t0:t1, :] = np.cumsum(x[:, t0:t1, :], axis=1)
    return out


def generate(w, *, B=None, T=None, H=None, K=None, seed=None, in_dtype=None,
             gate=None, beta=None, lengths=None) -> Inputs:
    """Draw the inputs of workload ``w`` (a Workload or its name).  Keyword
    overrides make variants of the same recipe (tests use them for small and
    edge-case shapes).  ``lengths`` gives explicit varlen sequence lengths."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    over = {k: v for k, v in dict(B=B, T=T, H=H, K=K, seed=seed, in_dtype=in_dtype,
                                    gate=gate, beta=beta).items() if v is not None}
    if lengths is not None:
        over["n_seqs"] = len(lengths)
        over["T"] = int(np.sum(lengths))
        over["B"] = 1
    if over:
        w = Workload(**{**w.__dict__, **over})
    rng = np.random.default_rng(w.seed)
    cu = None
    if w.n_seqs > 0:
        if w.B != 1:
            raise ValueError("varlen workloads have B == 1")
        lens = (np.asarray(lengths, dtype=np.int64) if lengths is not None
                else draw_lengths(rng, w.T, w.n_seqs, w.len_lo, w.len_hi))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        starts = cu.astype(np.int64)
    else:
        starts = np.array([0, w.T], dtype=np.int64)

    kk = rng.standard_normal((w.B, w.T, w.H, w.K))
    nrm = np.sqrt(np.sum(kk * kk, axis=-1, keepdims=True))
    kk /= nrm
    if w.in_dtype == "bf16":
        k_store = f64_to_bf16_bits(kk)
    elif w.in_dtype == "f16":
        k_store = kk.astype(np.float16).view(np.uint16)
    elif w.in_dtype == "f32":
        k_store = kk.astype(np.float32)
    else:
        raise ValueError(w.in_dtype)
    del kk

    b_arr = None
    if w.beta:
        u = rng.standard_normal((w.B, w.T, w.H))
        b_arr = (1.0 / (1.0 + np.exp(-u))).astype(np.float32)
    g_arr = g_raw = None
    if w.gate:
        u = rng.normal(4.0, 1.0, (w.B, w.T, w.H))
        logsig = -np.log1p(np.exp(-u))
        g_arr = chunk_local_cumsum(logsig, starts, w.T).astype(np.float32)
        g_raw = logsig.astype(np.float32)
    return Inputs(w, np.ascontiguousarray(k_store), g_arr, b_arr, cu, g_raw)


def chunk_geometry(T: int, cu_seqlens=None, chunk: int = CHUNK):
    """Per token: (local row index inside its chunk, chunk length).  Pure
    index bookkeeping, used by tests to build structural masks."""
    local = np.empty(T, dtype=np.int64)
    length = np.empty(T, dtype=np.int64)
    starts = [0, T] if cu_seqlens is None else list(np.asarray(cu_seqlens, dtype=np.int64))
    for s in range(len(starts) - 1):
        bos, eos = int(starts[s]), int(starts[s + 1])
        for t0 in range(bos, eos, chunk):
            t1 = min(t0 + chunk, eos)
            local[t0:t1] = np.arange(t1 - t0)
            length[t0:t1] = t1 - t0
    return local, length
