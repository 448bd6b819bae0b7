"""Comparison of a GPU result with the fp64 oracle (test infrastructure).

Acceptance criteria, element by element over the whole [B,T,H,64] output:
  * structure, bit-exact: no NaN anywhere (outputs are pre-filled with NaN, so
    this also proves every element was written); 1.0 on each row's diagonal;
    +0.0 (bit pattern 0) above the diagonal and in columns >= L;
  * fp32 output: max |gpu - ref| <= 2e-4 over all elements, and the mean
    relative error sum|gpu - ref| / sum|ref| over the strictly lower elements
    <= 1e-5;
  * bf16 / f16 output: each element within one unit in the last place of the
    format, measured as the distance in representable values between the GPU
    bits and the oracle's exact value rounded to nearest even, or
    |gpu - ref| <= 2^-23 (fp32 rounding of values near zero, where one bf16
    step is smaller than the fp32 arithmetic error);
  * f16 output only, when the caller passes the bound: an element may also
    lie within the first-order componentwise error of computing the inverse
    in fp32, c 2^-24 (|X| W |X|)[i, j] per chunk, where W >= |I + A|
    elementwise and c counts the roundings (see ``solve_bound``).  An f16 step
    is 8 times finer than a bf16 one, so where a row's terms cancel the fp32
    arithmetic error of the solve can exceed it.
"""
from __future__ import annotations

import numpy as np

import oracle
from chunked_gated_delta_token_amd import workloads

MAX_ABS_F32 = 2e-4
# Summed gate (the gate-sum entry point): within GATE_BOUND_ULPS 2^-24 of the
# running sum of |decay| (a 6-level fp32 tree sum has first-order error at
# most 6 2^-24 times that sum; 8 leaves room for the higher-order terms).
GATE_BOUND_ULPS = 8
MRE_F32 = 1e-5
FLOOR_16 = 2.0 ** -23
ONE_BITS = {"bf16": 0x3F80, "f16": 0x3C00}


def ordinal16(bits: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns to integers ordered like their values (+0 and -0 -> 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def decode(got: np.ndarray, out_dtype: str) -> np.ndarray:
    if out_dtype == "f32":
        return got.astype(np.float64)
    if out_dtype == "bf16":
        return workloads.bf16_bits_to_f64(got)
    return got.view(np.float16).astype(np.float64)


def structural_masks(T: int, cu_seqlens=None, chunk: int = 64):
    """[T, chunk] masks: diagonal, strictly upper (incl. columns >= L), strictly lower."""
    local, _length = workloads.chunk_geometry(T, cu_seqlens, chunk)
    j = np.arange(chunk)[None, :]
    i = local[:, None]
    return (j == i), (j > i), (j < i)


def compare(got: np.ndarray, ref: np.ndarray, out_dtype: str, cu_seqlens=None, label: str = "",
            bound=None) -> dict:
    """Assert the criteria above; return the measured figures.  The chunk
    size is the width of the rows (64 or 128).  ``bound`` is None or a
    callable returning the [B,T,H,C] fp32 error bound of each element (f16
    output only; evaluated only when some element is beyond 1 ulp)."""
    B, T, H, C = ref.shape
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diag, upper, lower = (m[None, :, None, :] for m in structural_masks(T, cu_seqlens, C))
    diag = np.broadcast_to(diag, ref.shape)
    upper = np.broadcast_to(upper, ref.shape)
    lower = np.broadcast_to(lower, ref.shape)
    val = decode(got, out_dtype)
    stats = {"label": label, "elements": int(ref.size)}
    assert not np.any(np.isnan(val)), f"{label}: NaN in output (unwritten elements?)"
    if out_dtype == "f32":
        bits = got.view(np.uint32)
        assert np.all(val[diag] == 1.0), f"{label}: diagonal is not exactly 1.0"
        assert np.all(bits[upper] == 0), f"{label}: upper triangle is not +0.0"
        err = np.abs(val - ref)
        max_abs = float(err.max())
        mre = float(err[lower].sum() / max(np.abs(ref[lower]).sum(), 1e-300))
        stats.update(max_abs=max_abs, mre=mre)
        assert max_abs <= MAX_ABS_F32, f"{label}: max abs error {max_abs:.3e} > {MAX_ABS_F32}"
        assert mre <= MRE_F32, f"{label}: mean relative error {mre:.3e} > {MRE_F32}"
    else:
        assert np.all(got[diag] == ONE_BITS[out_dtype]), f"{label}: diagonal is not exactly 1.0"
        assert np.all(got[upper] == 0), f"{label}: upper triangle is not +0.0"
        exp_bits = oracle.round_to_bf16_bits(ref) if out_dtype == "bf16" else oracle.round_to_f16_bits(ref)
        dist = np.abs(ordinal16(got) - ordinal16(exp_bits))
        err = np.abs(val - ref)
        ok_ulp = dist <= 1
        ok_floor = err <= FLOOR_16
        bad = ~(ok_ulp | ok_floor)
        stats.update(max_ulp=int(dist.max()), n_floor=int(np.sum(~ok_ulp & ok_floor)),
                     max_abs=float(err.max()), exact_frac=float(np.mean(dist == 0)))
        if out_dtype == "f16" and bound is not None and np.any(bad):
            b = bound()
            ok_bound = bad & (err <= b)
            stats.update(n_bound=int(ok_bound.sum()),
                         max_err_over_bound=float(np.max(err[bad] / np.maximum(b[bad], 1e-300))))
            bad &= ~ok_bound
        assert not np.any(bad), (f"{label}: {int(bad.sum())} elements beyond 1 ulp "
                                 f"(max {int(dist.max())} ulp, first at {np.argwhere(bad)[0].tolist()})")
    return stats


# ---------------------------------------------------------------- A (first step of the unfused chain)
U32 = 2.0 ** -24          # unit roundoff of fp32
GATE_ULPS = 128           # exp of a gate difference of magnitude <= 50, see compare_A


def a_scale(k64: np.ndarray, g, beta, cu_seqlens=None, chunk: int = 64) -> np.ndarray:
    """Per element of A, the magnitude its rounding errors are relative to:
    |beta_i| * sum_k |k_ik k_jk| * exp(clamp(g_i - g_j)), i.e. the oracle's A
    of |k| and |beta| (an upper bound of |A| whose terms are all positive)."""
    return oracle.scaled_dot_ref(np.abs(k64), g, None if beta is None else np.abs(beta), cu_seqlens,
                                 chunk_size=chunk)


def solve_bound(X: np.ndarray, W: np.ndarray, c: float, cu_seqlens=None) -> np.ndarray:
    """c 2^-24 (|X| (I + W) |X|) for every chunk and head, laid out like X
    ([B,T,H,C], row t holding its chunk's row; zero outside each chunk).

    Computing the inverse X of a unit lower triangular M by substitution in
    fp32 gives, to first order, |X^ - X| <= n u |X||M||X| (Higham, Accuracy
    and Stability of Numerical Algorithms, ch. 8, the componentwise backward
    error of substitution applied to each column of M X = I).  An error
    |dA| <= e u W made in forming A adds at most e u |X| W |X|.  With
    |M| <= I + W both fold into c u |X| (I + W) |X|, c = n + e."""
    B, T, H, C = X.shape
    local, length = workloads.chunk_geometry(T, cu_seqlens, C)
    out = np.zeros_like(X, dtype=np.float64)
    for t0 in np.nonzero(local == 0)[0]:
        L = int(length[t0])
        xa = np.abs(X[:, t0:t0 + L, :, :L]).transpose(0, 2, 1, 3)          # [B, H, L, L]
        m = np.eye(L) + np.abs(W[:, t0:t0 + L, :, :L]).transpose(0, 2, 1, 3)
        out[:, t0:t0 + L, :, :L] = (xa @ m @ xa).transpose(0, 2, 1, 3)
    return c * U32 * out


def fused_bound(inp, ref: np.ndarray, chunk: int = 64, gate_err: float = 0.0):
    """The ``bound`` argument of ``compare`` for the fused op on ``inp``:
    W = a_scale (>= |A|), c = chunk + K + GATE_ULPS (the solve's inner
    products, then A's dot product and gate as in ``compare_A``) + gate_err
    (the error of a summed gate, in units of 2^-24 per unit of exp's
    argument)."""
    def make():
        W = a_scale(inp.k64(), inp.g, inp.beta, inp.cu_seqlens, chunk)
        return solve_bound(ref, W, chunk + inp.workload.K + GATE_ULPS + gate_err, inp.cu_seqlens)
    return make


def tril_bound(A: np.ndarray, ref: np.ndarray, cu_seqlens=None):
    """The ``bound`` argument of ``compare`` for the solve of a given fp32 A
    (exact input, so only the solve's own roundings: c = chunk size).  Only
    the strictly lower part of each chunk of A is read."""
    def make():
        C = ref.shape[3]
        _d, _u, lower = structural_masks(ref.shape[1], cu_seqlens, C)
        W = np.where(np.broadcast_to(lower[None, :, None, :], A.shape), np.abs(A.astype(np.float64)), 0.0)
        return solve_bound(ref, W, C, cu_seqlens)
    return make


def compare_A(got: np.ndarray, ref: np.ndarray, scale: np.ndarray, K: int, cu_seqlens=None,
              label: str = "") -> dict:
    """A in fp32 against the oracle's fp64 A.

    Structure, bit-exact: +0.0 on and above the diagonal and in columns >= L.
    Strictly lower elements: |gpu - ref| <= (K + 128) 2^-24 scale.  K 2^-24
    bounds an fp32 dot product of length K (products of 16-bit inputs are
    exact in fp32; fp32 inputs are summed as six products of their three-part
    bf16 splits, whose split error and left-out terms stay below 2^-25 of
    each |k_ik k_jk|, within the same bound); 128 2^-24 covers the gate: the difference g_i - g_j (or g_i - g_0
    and g_0 - g_j, |.| <= 25, in the factored form) rounds with an absolute
    error up to 50 2^-24, exp turns that into the same relative error, and the
    exp2 instruction with its scaling by log2(e) adds about as much again, plus
    the few products with beta.
    """
    B, T, H, C = ref.shape
    assert got.shape == ref.shape, (got.shape, ref.shape)
    _diag, upper, lower = (np.broadcast_to(m[None, :, None, :], ref.shape)
                           for m in structural_masks(T, cu_seqlens))
    zero_region = ~lower
    stats = {"label": label, "elements": int(ref.size)}
    assert not np.any(np.isnan(got)), f"{label}: NaN in A (unwritten elements?)"
    assert np.all(got.view(np.uint32)[zero_region] == 0), f"{label}: A is not +0.0 on/above the diagonal"
    err = np.abs(got.astype(np.float64) - ref)
    bound = (K + GATE_ULPS) * U32 * scale
    ratio = np.where(lower, err / np.maximum(bound, 1e-300), 0.0)
    stats.update(max_err_over_bound=float(ratio.max()),
                 max_rel_to_scale=float(np.max(np.where(lower, err / np.maximum(scale, 1e-300), 0.0))))
    bad = lower & (err > bound)
    assert not np.any(bad), (f"{label}: {int(bad.sum())} elements of A beyond (K+128) 2^-24 scale, "
                             f"worst ratio {stats['max_err_over_bound']:.2f} at {np.argwhere(bad)[0].tolist()}")
    return stats
