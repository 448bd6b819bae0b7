"""Pins for the fp64 oracle: checks against facts fixed by the pages and by
mathematics, not against the oracle's own formula.

Each ``pin_*`` takes ``solve`` (a callable with the signature of
``oracle.kkt_solve_ref``) and raises AssertionError if the oracle it is given
is wrong.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and requires every mistake to fail at least one pin.

Definition pinned (MindSpeed-Ops PR #135 page, "feat(triton): add
chunk_gated_delta_rule_fwd_kkt_solve": PR description, user-facing-change
section, bot change summary): per 64-token chunk,
A[i][j] = beta_i (k_i . k_j) exp(clamp(g_i - g_j, -50, 50)) for i > j, and the
output rows are those of (I + A)^{-1}.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked_chunks.json")
CH = 64


def _unit_keys(rng, B, T, H, K):
    k = rng.standard_normal((B, T, H, K))
    return k / np.linalg.norm(k, axis=-1, keepdims=True)


def _decay(rng, B, T, H, scale=1.0):
    """A chunk-local cumsum of negative increments (a valid log-decay)."""
    inc = -scale * rng.uniform(0.0, 0.2, (B, T, H))
    g = np.empty_like(inc)
    for t0 in range(0, T, CH):
        g[:, t0:t0 + CH] = np.cumsum(inc[:, t0:t0 + CH], axis=1)
    return g


# --------------------------------------------------------------------------
# Hand-worked golden chunks (values derived by hand, file carries the steps)
# --------------------------------------------------------------------------
def pin_golden(solve):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        k = np.array(c["k"], dtype=np.float64)
        T, K = k.shape
        k = k.reshape(1, T, 1, K)
        beta = None if c["beta"] is None else np.array(c["beta"]).reshape(1, T, 1)
        g = None if c["g"] is None else np.array(c["g"]).reshape(1, T, 1)
        cu = None if c["cu_seqlens"] is None else np.array(c["cu_seqlens"], dtype=np.int32)
        out = solve(k, g, beta, cu)
        assert out.shape == (1, T, 1, CH), c["name"]
        for t, row in enumerate(c["expected_rows"]):
            exp = np.zeros(CH)
            exp[:len(row)] = row
            got = out[0, t, 0]
            if "tol_rel" in c:
                ok = np.all(np.abs(got - exp) <= c["tol_rel"] * np.maximum(np.abs(exp), 1.0))
            else:
                ok = np.all(np.abs(got - exp) <= c["tol"])
            assert ok, f"{c['name']} row {t}: got {got[:4]} expected {exp[:4]}"


# --------------------------------------------------------------------------
# P-a: 2x2 and 3x3 brute force on exact rationals
# --------------------------------------------------------------------------
def _exact_inverse(M):
    """Inverse of a small matrix of Fractions by the adjugate (cofactor) rule."""
    n = len(M)

    def det(m):
        if len(m) == 1:
            return m[0][0]
        return sum(((-1) ** c) * m[0][c] * det([row[:c] + row[c + 1:] for row in m[1:]])
                   for c in range(len(m)))

    d = det(M)
    inv = [[None] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            minor = [row[:i] + row[i + 1:] for r, row in enumerate(M) if r != j]
            inv[i][j] = ((-1) ** (i + j)) * (det(minor) if minor else Fraction(1)) / d
    return inv


def pin_bruteforce_small(solve):
    """Integer keys, dyadic beta, no gate: the exact inverse over the
    rationals by the cofactor rule must match to fp64 rounding."""
    rng = np.random.default_rng(11)
    for T in (2, 3):
        for _ in range(5):
            K = 3
            ki = rng.integers(-3, 4, size=(T, K))
            bi = rng.integers(1, 8, size=T)  # beta = bi / 8
            M = [[Fraction(int(i == j)) for j in range(T)] for i in range(T)]
            for i in range(T):
                for j in range(i):
                    M[i][j] = Fraction(int(bi[i]), 8) * int(np.dot(ki[i], ki[j]))
            X = _exact_inverse(M)
            out = solve(ki.reshape(1, T, 1, K).astype(np.float64), None,
                        (bi / 8.0).reshape(1, T, 1), None)
            for i in range(T):
                for j in range(CH):
                    exp = float(X[i][j]) if j < T else 0.0
                    assert abs(out[0, i, 0, j] - exp) <= 1e-12 * max(1.0, abs(exp)), (T, i, j)


# --------------------------------------------------------------------------
# P-b: identical unit keys -> closed form
#   X[i][j] = -beta_i exp(g_i - g_j) prod_{m=j+1}^{i-1} (1 - beta_m), i > j
# --------------------------------------------------------------------------
def pin_identical_keys_closed_form(solve):
    rng = np.random.default_rng(12)
    for T, H, K in ((64, 2, 4), (47, 1, 8), (130, 3, 2)):
        k = np.zeros((1, T, H, K))
        k[..., 0] = 1.0
        beta = rng.uniform(0.05, 0.95, (1, T, H))
        g = _decay(rng, 1, T, H, scale=3.5)  # within-chunk spread up to ~44 (< 50: clamp never binds)
        out = solve(k, g, beta, None)
        for h in range(H):
            for t0 in range(0, T, CH):
                L = min(CH, T - t0)
                b = beta[0, t0:t0 + L, h]
                gg = g[0, t0:t0 + L, h]
                for i in range(L):
                    for j in range(CH):
                        if j == i:
                            exp = 1.0
                        elif j < i:
                            d = np.clip(gg[i] - gg[j], -50.0, 50.0)
                            exp = -b[i] * np.exp(d) * np.prod(1.0 - b[j + 1:i])
                        else:
                            exp = 0.0
                        got = out[0, t0 + i, h, j]
                        assert abs(got - exp) <= 1e-10 * abs(exp) + 1e-15, (T, h, t0, i, j, got, exp)


# --------------------------------------------------------------------------
# P-c: the gate is a diagonal similarity, X(g) = D X(0) D^{-1}, D = diag(e^g)
# --------------------------------------------------------------------------
def pin_gate_similarity(solve):
    rng = np.random.default_rng(13)
    B, T, H, K = 2, 128, 3, 16
    k = _unit_keys(rng, B, T, H, K)
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    g = _decay(rng, B, T, H, scale=2.0)
    x_g = solve(k, g, beta, None)
    x_0 = solve(k, None, beta, None)
    for t0 in range(0, T, CH):
        sl = slice(t0, t0 + CH)
        d = np.exp(g[:, sl, :])                     # [B, L, H]
        # D X(0) D^{-1}: row i scaled by e^{g_i}, column j by e^{-g_j}
        expect = d[..., None] * x_0[:, sl, :, :] / np.transpose(d, (0, 2, 1))[:, None, :, :]
        assert np.allclose(x_g[:, sl], expect, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# P-d / P-e / P-f: structure
# --------------------------------------------------------------------------
def pin_orthogonal_keys_identity(solve):
    T, K = 64, 64
    k = np.zeros((1, T, 2, K))
    for t in range(T):
        k[0, t, :, t] = 1.0
    rng = np.random.default_rng(14)
    out = solve(k, _decay(rng, 1, T, 2), rng.uniform(0.1, 0.9, (1, T, 2)), None)
    assert np.array_equal(out[0, :, 0, :], np.eye(T))
    assert np.array_equal(out[0, :, 1, :], np.eye(T))


def pin_beta_zero(solve):
    rng = np.random.default_rng(15)
    T, H, K = 100, 2, 8
    k = _unit_keys(rng, 1, T, H, K)
    g = _decay(rng, 1, T, H)
    out = solve(k, g, np.zeros((1, T, H)), None)
    local = np.arange(T) % CH
    for t in range(T):
        e = np.zeros(CH)
        e[local[t]] = 1.0
        assert np.array_equal(out[0, t, 0], e) and np.array_equal(out[0, t, 1], e)
    # one row with beta = 0: that row is e_i
    beta = rng.uniform(0.2, 0.9, (1, T, H))
    beta[0, 70, 1] = 0.0
    out = solve(k, g, beta, None)
    e = np.zeros(CH)
    e[70 - 64] = 1.0
    assert np.array_equal(out[0, 70, 1], e)
    assert not np.array_equal(out[0, 70, 0], e)


def pin_single_token(solve):
    rng = np.random.default_rng(16)
    out = solve(_unit_keys(rng, 1, 1, 3, 8), _decay(rng, 1, 1, 3), rng.uniform(size=(1, 1, 3)), None)
    e = np.zeros(CH)
    e[0] = 1.0
    for h in range(3):
        assert np.array_equal(out[0, 0, h], e)


# --------------------------------------------------------------------------
# P-g: residual and unit lower triangle.  A is written out here from the
# definition only to form the residual (I + A) X - I.
# --------------------------------------------------------------------------
def pin_residual(solve):
    rng = np.random.default_rng(17)
    B, T, H, K = 1, 150, 2, 32
    k = _unit_keys(rng, B, T, H, K)
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    g = _decay(rng, B, T, H)
    out = solve(k, g, beta, None)
    for h in range(H):
        for t0 in range(0, T, CH):
            L = min(CH, T - t0)
            kk = k[0, t0:t0 + L, h]
            gg = g[0, t0:t0 + L, h]
            A = np.tril(beta[0, t0:t0 + L, h][:, None] * (kk @ kk.T)
                        * np.exp(np.clip(gg[:, None] - gg[None, :], -50, 50)), -1)
            X = out[0, t0:t0 + L, h, :L]
            assert np.max(np.abs((np.eye(L) + A) @ X - np.eye(L))) <= 1e-12
            assert np.max(np.abs(np.triu(X, 1))) <= 1e-12
            assert np.max(np.abs(np.diag(X) - 1.0)) <= 1e-12
            assert np.all(out[0, t0:t0 + L, h, L:] == 0.0)


# --------------------------------------------------------------------------
# P-h: no gate, no beta reduces to (I + strict_tril(K K^T))^{-1}: checked
# against numpy.linalg.inv and against a separate forward substitution.
# --------------------------------------------------------------------------
def _forward_substitution_inverse(M):
    n = M.shape[0]
    X = np.zeros_like(M)
    for c in range(n):
        for r in range(n):
            X[r, c] = ((r == c) - M[r, :r] @ X[:r, c]) / M[r, r]
    return X


def pin_plain_kkt_library_inverse(solve):
    rng = np.random.default_rng(18)
    T, H, K = 200, 3, 64
    k = _unit_keys(rng, 1, T, H, K)
    out = solve(k, None, None, None)
    for h in range(H):
        for t0 in range(0, T, CH):
            L = min(CH, T - t0)
            kk = k[0, t0:t0 + L, h]
            M = np.eye(L) + np.tril(kk @ kk.T, -1)
            ref = np.linalg.inv(M)
            fs = _forward_substitution_inverse(M)
            got = out[0, t0:t0 + L, h, :L]
            scale = max(1.0, np.max(np.abs(ref)))
            assert np.max(np.abs(got - ref)) <= 1e-13 * scale
            assert np.max(np.abs(got - fs)) <= 1e-13 * scale


# --------------------------------------------------------------------------
# P-i: independence of chunks, heads, batch rows and sequences
# --------------------------------------------------------------------------
def pin_equivariance(solve):
    rng = np.random.default_rng(19)
    B, T, H, K = 2, 192, 3, 16
    k = _unit_keys(rng, B, T, H, K)
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    g = _decay(rng, B, T, H)
    base = solve(k, g, beta, None)
    # heads
    p = np.array([2, 0, 1])
    assert np.array_equal(solve(k[:, :, p], g[:, :, p], beta[:, :, p], None), base[:, :, p])
    # batch rows
    assert np.array_equal(solve(k[::-1], g[::-1], beta[::-1], None), base[::-1])
    # whole chunks (g is chunk-local, so chunks are self-contained)
    order = np.concatenate([np.arange(128, 192), np.arange(0, 64), np.arange(64, 128)])
    assert np.array_equal(solve(k[:, order], g[:, order], beta[:, order], None), base[:, order])


def pin_varlen_is_concat(solve):
    """A packed batch equals separate fixed-length calls per sequence (the
    pages test varlen by splitting cu_seqlens into segments)."""
    rng = np.random.default_rng(20)
    lens = [70, 1, 0, 64, 129, 3, 0]
    T, H, K = sum(lens), 2, 16
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    k = _unit_keys(rng, 1, T, H, K)
    beta = rng.uniform(0.1, 0.9, (1, T, H))
    g = np.empty((1, T, H))
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if b > a:
            g[:, a:b] = _decay(rng, 1, b - a, H)
    out = solve(k, g, beta, cu)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        ref = solve(k[:, a:b], g[:, a:b], beta[:, a:b], None)
        assert np.array_equal(out[:, a:b], ref), s


# --------------------------------------------------------------------------
# P-j: a per-chunk constant added to g changes nothing
# --------------------------------------------------------------------------
def pin_gate_shift_invariance(solve):
    rng = np.random.default_rng(21)
    B, T, H, K = 1, 192, 2, 16
    k = _unit_keys(rng, B, T, H, K)
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    g = _decay(rng, B, T, H)
    shift = np.repeat(rng.uniform(-5, 5, (B, T // CH, H)), CH, axis=1)
    a = solve(k, g, beta, None)
    b = solve(k, g + shift, beta, None)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# P-k: prefix property (a partial last chunk equals the first rows of a full one)
# --------------------------------------------------------------------------
def pin_prefix(solve):
    rng = np.random.default_rng(22)
    B, T, H, K = 1, 128, 2, 16
    k = _unit_keys(rng, B, T, H, K)
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    g = _decay(rng, B, T, H)
    full = solve(k, g, beta, None)
    for Tp in (65, 100, 127):
        part = solve(k[:, :Tp], g[:, :Tp], beta[:, :Tp], None)
        L = Tp - 64
        assert np.allclose(part[:, :64], full[:, :64], rtol=0, atol=0)
        assert np.allclose(part[:, 64:, :, :L], full[:, 64:Tp, :, :L], rtol=1e-13, atol=1e-15)
        assert np.all(part[:, 64:, :, L:] == 0.0)


# --------------------------------------------------------------------------
# P-l: g = 0 and beta = 1 are the same as no gate / no beta
# --------------------------------------------------------------------------
def pin_neutral_gate_beta(solve):
    rng = np.random.default_rng(23)
    B, T, H, K = 1, 96, 2, 16
    k = _unit_keys(rng, B, T, H, K)
    a = solve(k, None, None, None)
    b = solve(k, np.zeros((B, T, H)), np.ones((B, T, H)), None)
    assert np.array_equal(a, b)


ALL_PINS = [
    pin_golden,
    pin_bruteforce_small,
    pin_identical_keys_closed_form,
    pin_gate_similarity,
    pin_orthogonal_keys_identity,
    pin_beta_zero,
    pin_single_token,
    pin_residual,
    pin_plain_kkt_library_inverse,
    pin_equivariance,
    pin_varlen_is_concat,
    pin_gate_shift_invariance,
    pin_prefix,
    pin_neutral_gate_beta,
]


# --------------------------------------------------------------------------
# The two steps of the unfused chain on their own.  These pins take
# (solve, scaled_dot, solve_tril).
# --------------------------------------------------------------------------
def split_pin_golden_A(solve, scaled_dot, solve_tril):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        k = np.array(c["k"], dtype=np.float64)
        T, K = k.shape
        k = k.reshape(1, T, 1, K)
        beta = None if c["beta"] is None else np.array(c["beta"]).reshape(1, T, 1)
        g = None if c["g"] is None else np.array(c["g"]).reshape(1, T, 1)
        cu = None if c["cu_seqlens"] is None else np.array(c["cu_seqlens"], dtype=np.int32)
        A = scaled_dot(k, g, beta, cu)
        for t, row in enumerate(c["expected_A_rows"]):
            exp = np.zeros(CH)
            exp[:len(row)] = row
            tol = c.get("tol", 0.0) + c.get("tol_rel", 0.0) * np.abs(exp)
            assert np.all(np.abs(A[0, t, 0] - exp) <= tol), (c["name"], t, A[0, t, 0, :4])


def split_pin_solve_tril_library_inverse(solve, scaled_dot, solve_tril):
    """Random strictly lower A against numpy.linalg.inv(I + A), chunk by chunk;
    whatever sits on or above A's diagonal is ignored."""
    rng = np.random.default_rng(40)
    B, T, H = 2, 150, 3
    A = rng.uniform(-0.3, 0.3, (B, T, H, CH))
    garbage = A.copy()
    for t in range(T):
        i = t % CH
        A[:, t, :, i:] = 0.0
        garbage[:, t, :, i:] = rng.uniform(-50, 50, (B, H, CH - i))
    X = solve_tril(A)
    assert np.array_equal(solve_tril(garbage), X)
    for b in range(B):
        for h in range(H):
            for t0 in range(0, T, CH):
                L = min(CH, T - t0)
                ref = np.linalg.inv(np.eye(L) + A[b, t0:t0 + L, h, :L])
                got = X[b, t0:t0 + L, h, :L]
                assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))
                assert np.all(X[b, t0:t0 + L, h, L:] == 0.0)


def split_pin_composition(solve, scaled_dot, solve_tril):
    """solve_tril(scaled_dot(x)) is the fused result, bit for bit, also for
    packed sequences (the pages' fused op equals the two-step chain)."""
    rng = np.random.default_rng(41)
    lens = [70, 1, 0, 129, 3]
    T, H, K = sum(lens), 2, 16
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    k = _unit_keys(rng, 1, T, H, K)
    beta = rng.uniform(0.1, 0.9, (1, T, H))
    g = -np.cumsum(rng.uniform(0, 0.1, (1, T, H)), axis=1)
    for cu_ in (None, cu):
        assert np.array_equal(solve_tril(scaled_dot(k, g, beta, cu_), cu_), solve(k, g, beta, cu_))


SPLIT_PINS = [split_pin_golden_A, split_pin_solve_tril_library_inverse, split_pin_composition]


# --------------------------------------------------------------------------
# The gate from the per-token log-decay: g is its running sum restarted at
# every chunk.  These pins take (solve, cumsum), cumsum with the signature of
# oracle.chunk_cumsum_ref.
# --------------------------------------------------------------------------
def _local_index(T, cu, chunk):
    """Row index inside its chunk, counted from each sequence start."""
    starts = [0, T] if cu is None else [int(x) for x in cu]
    local = np.zeros(T, dtype=np.int64)
    for s in range(len(starts) - 1):
        for t in range(starts[s], starts[s + 1]):
            local[t] = (t - starts[s]) % chunk
    return local


def cumsum_pin_constant_closed_form(solve, cumsum):
    """A constant decay c gives g = c (i + 1) at local row i (exact in fp64
    for c = -0.25 and i < 64), per batch row and per packed sequence."""
    c = -0.25
    for B, T, cu in ((2, 150, None), (1, 143, np.array([0, 5, 75, 75, 78, 142, 143], dtype=np.int32))):
        H = 3
        g = cumsum(np.full((B, T, H), c), cu)
        exp = c * (_local_index(T, cu, CH) + 1.0)
        assert np.array_equal(g, np.broadcast_to(exp[None, :, None], g.shape)), (B, T)


def cumsum_pin_bruteforce(solve, cumsum):
    """Random decays, small chunk sizes: every g[t] equals the explicit sum of
    the decays from its chunk's first row to t."""
    rng = np.random.default_rng(50)
    for B, T, H, chunk, cu in ((2, 13, 2, 4, None),
                               (1, 11, 3, 3, np.array([0, 2, 2, 9, 11], dtype=np.int32))):
        a = rng.uniform(-1.0, 0.0, (B, T, H))
        g = cumsum(a, cu, chunk)
        local = _local_index(T, cu, chunk)
        for b in range(B):
            for t in range(T):
                for h in range(H):
                    ref = 0.0
                    for s in range(t - local[t], t + 1):
                        ref += a[b, s, h]
                    assert abs(g[b, t, h] - ref) <= 1e-15 * max(1.0, abs(ref)), (b, t, h)


def cumsum_pin_first_row_irrelevant(solve, cumsum):
    """Only the differences g_i - g_j (i > j) enter A, and they sum the decays
    of rows j+1 .. i: the decay of each chunk's first row changes nothing,
    the decay of any other row does."""
    rng = np.random.default_rng(51)
    B, T, H, K = 1, 150, 2, 16
    k = _unit_keys(rng, B, T, H, K)
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    a = rng.uniform(-0.2, 0.0, (B, T, H))
    base = solve(k, cumsum(a), beta, None)
    first = a.copy()
    first[:, ::CH] = rng.uniform(-3.0, 3.0, first[:, ::CH].shape)
    assert np.allclose(solve(k, cumsum(first), beta, None), base, rtol=1e-12, atol=1e-13)
    other = a.copy()
    other[:, 1::CH] -= 0.5
    assert not np.allclose(solve(k, cumsum(other), beta, None), base, rtol=1e-6, atol=1e-8)


CUMSUM_PINS = [cumsum_pin_constant_closed_form, cumsum_pin_bruteforce, cumsum_pin_first_row_irrelevant]


# --------------------------------------------------------------------------
# Chunks of 128 tokens (the chunk size of the GDR case page's tiling).  These
# pins take solve (with a chunk_size keyword) and hold the 128-token result to
# the 64-token one, which the pins above fix.
# --------------------------------------------------------------------------
def _A_block(k, g, beta, rows, cols):
    """beta_i (k_i . k_j) exp(clamp(g_i - g_j)) for token rows x token cols
    (one batch row, one head)."""
    G = np.clip(g[rows][:, None] - g[cols][None, :], -50.0, 50.0)
    return beta[rows][:, None] * (k[rows] @ k[cols].T) * np.exp(G)


def chunk128_pin_block_inverse(solve):
    """Split a 128-token chunk into halves: the diagonal blocks of its inverse
    are the 64-token results of each half, the upper block is zero, and the
    lower block is -X22 A21 X11 (the inverse of a block lower-triangular
    matrix).  Covers a full chunk and a partial one (T = 2*128 + 100)."""
    rng = np.random.default_rng(60)
    B, T, H, K = 1, 356, 2, 16
    k = _unit_keys(rng, B, T, H, K)
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    g = np.empty((B, T, H))
    for t0 in range(0, T, 128):
        g[:, t0:t0 + 128] = np.cumsum(-rng.uniform(0.0, 0.1, g[:, t0:t0 + 128].shape), axis=1)
    X = solve(k, g, beta, None, chunk_size=128)
    assert X.shape == (B, T, H, 128)
    for t0 in range(0, T, 128):
        L = min(128, T - t0)
        L2 = L - 64
        top = solve(k[:, t0:t0 + 64], g[:, t0:t0 + 64], beta[:, t0:t0 + 64], None)
        bot = solve(k[:, t0 + 64:t0 + L], g[:, t0 + 64:t0 + L], beta[:, t0 + 64:t0 + L], None)
        for h in range(H):
            X11 = top[0, :, h, :64]
            X22 = bot[0, :, h, :L2]
            A21 = _A_block(k[0, :, h], g[0, :, h], beta[0, :, h],
                           np.arange(t0 + 64, t0 + L), np.arange(t0, t0 + 64))
            X21 = -X22 @ A21 @ X11
            got = X[0, t0:t0 + L, h]
            tol = 1e-12 * max(1.0, np.max(np.abs(X21)))
            assert np.max(np.abs(got[:64, :64] - X11)) <= tol
            assert np.all(got[:64, 64:] == 0.0)
            assert np.max(np.abs(got[64:, 64:L] - X22)) <= tol
            assert np.max(np.abs(got[64:, :64] - X21)) <= tol
            assert np.all(got[:, L:] == 0.0)


def chunk128_pin_library_inverse(solve):
    """No gate, no beta: each 128-token chunk is numpy.linalg.inv(I + strict
    lower part of K K^T)."""
    rng = np.random.default_rng(61)
    B, T, H, K = 2, 200, 1, 32
    k = _unit_keys(rng, B, T, H, K)
    X = solve(k, None, None, None, chunk_size=128)
    for b in range(B):
        for t0 in range(0, T, 128):
            L = min(128, T - t0)
            kk = k[b, t0:t0 + L, 0]
            ref = np.linalg.inv(np.eye(L) + np.tril(kk @ kk.T, -1))
            assert np.max(np.abs(X[b, t0:t0 + L, 0, :L] - ref)) <= 1e-11 * max(1.0, np.max(np.abs(ref)))


def chunk128_pin_varlen_is_concat(solve):
    """Packed sequences at chunk 128 equal one call per sequence; chunks
    restart at every sequence start."""
    rng = np.random.default_rng(62)
    lens = [130, 1, 0, 128, 257, 64]
    T, H, K = sum(lens), 2, 16
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    k = _unit_keys(rng, 1, T, H, K)
    beta = rng.uniform(0.1, 0.9, (1, T, H))
    g = -np.cumsum(rng.uniform(0.0, 0.05, (1, T, H)), axis=1)
    out = solve(k, g, beta, cu, chunk_size=128)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if b > a:
            ref = solve(k[:, a:b], g[:, a:b], beta[:, a:b], None, chunk_size=128)
            assert np.array_equal(out[:, a:b], ref), s


CHUNK128_PINS = [chunk128_pin_block_inverse, chunk128_pin_library_inverse, chunk128_pin_varlen_is_concat]
