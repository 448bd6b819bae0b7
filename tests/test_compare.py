"""The acceptance criteria of the GPU tests, exercised on the CPU: the
oracle's own results rounded as a kernel would round them pass, and the
mistakes the criteria exist for (an unwritten element, a nonzero where the
output must be +0.0, an error beyond the bound) fail."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from chunked_gated_delta_token_amd import workloads as W
from tests._compare import GATE_ULPS, U32, a_scale, compare, compare_A, fused_bound, solve_bound


@pytest.fixture(scope="module")
def case():
    inp = W.generate("T256_H8_bf16_f32", T=150, H=2, seed=900)
    k64 = inp.k64()
    A = oracle.scaled_dot_ref(k64, inp.g, inp.beta)
    return inp, A, a_scale(k64, inp.g, inp.beta)


def test_scale_bounds_A(case):
    _inp, A, scale = case
    assert np.all(np.abs(A) <= scale * (1 + 1e-12))


def test_compare_A_accepts_fp32_rounding(case):
    inp, A, scale = case
    stats = compare_A(A.astype(np.float32), A, scale, inp.workload.K)
    assert stats["max_err_over_bound"] < 0.01


def test_compare_A_rejects_mistakes(case):
    inp, A, scale = case
    K = inp.workload.K
    got = A.astype(np.float32)
    i = np.argwhere((A != 0))[-1]
    bad = got.copy()
    bad[tuple(i)] += np.float32(3 * (K + GATE_ULPS) * U32 * scale[tuple(i)])
    with pytest.raises(AssertionError):
        compare_A(bad, A, scale, K)
    bad = got.copy()
    bad[0, 3, 1, 3] = 1e-30  # diagonal must be +0.0
    with pytest.raises(AssertionError):
        compare_A(bad, A, scale, K)
    bad = got.copy()
    bad[0, 3, 1, 5] = -0.0  # upper part must be +0.0, not -0.0
    with pytest.raises(AssertionError):
        compare_A(bad, A, scale, K)
    bad = got.copy()
    bad[0, 149, 0, 10] = np.nan  # unwritten element
    with pytest.raises(AssertionError):
        compare_A(bad, A, scale, K)


def test_compare_accepts_rounded_inverse_and_rejects_mistakes(case):
    inp, _A, _s = case
    X = oracle.kkt_solve_ref(inp.k64(), inp.g, inp.beta)
    compare(X.astype(np.float32), X, "f32")
    compare(oracle.round_to_bf16_bits(X), X, "bf16")
    compare(oracle.round_to_f16_bits(X), X, "f16")
    bad = X.astype(np.float32)
    bad[0, 70, 1, 3] += 1e-3
    with pytest.raises(AssertionError):
        compare(bad, X, "f32")
    bad = oracle.round_to_bf16_bits(X)
    bad[0, 70, 1, 3] += 2  # two bf16 steps
    with pytest.raises(AssertionError):
        compare(bad, X, "bf16")
    bad = X.astype(np.float32)
    bad[0, 70, 1, 6] = 1.0  # diagonal position of row 70 is column 6
    bad[0, 70, 1, 7] = 1e-20  # above the diagonal
    with pytest.raises(AssertionError):
        compare(bad, X, "f32")


# ---------------------------------------------------------------- the fp32 solve bound (f16 output)
def _fp32_inverse(inp: W.Inputs, chunk: int) -> np.ndarray:
    """A plain fp32 computation of the same rows, independent of the kernels:
    A formed in fp32, each chunk's rows by forward substitution in fp32."""
    k = inp.k64().astype(np.float32)
    B, T, H, _K = k.shape
    local, length = W.chunk_geometry(T, inp.cu_seqlens, chunk)
    out = np.zeros((B, T, H, chunk), np.float32)
    for t0 in np.nonzero(local == 0)[0]:
        L = int(length[t0])
        kk = k[:, t0:t0 + L].transpose(0, 2, 1, 3)                          # [B, H, L, K]
        a = kk @ kk.transpose(0, 1, 3, 2)
        if inp.g is not None:
            g = inp.g[:, t0:t0 + L].transpose(0, 2, 1).astype(np.float32)
            a = a * np.exp(np.clip(g[..., :, None] - g[..., None, :], -50, 50))
        if inp.beta is not None:
            a = a * inp.beta[:, t0:t0 + L].transpose(0, 2, 1)[..., :, None].astype(np.float32)
        a = np.tril(a, -1).astype(np.float32)
        y = np.zeros_like(a)
        for i in range(L):
            row = -np.einsum("bhj,bhjc->bhc", a[:, :, i, :i], y[:, :, :i, :]).astype(np.float32)
            row[..., i] = 1.0
            row[..., i + 1:] = 0.0
            y[:, :, i, :] = row
        out[:, t0:t0 + L, :, :L] = y.transpose(0, 2, 1, 3)
    return out


@pytest.mark.parametrize("chunk", [64, 128])
def test_solve_bound_layout(chunk):
    """solve_bound against the sum written out element by element, on packed
    sequences with partial chunks."""
    inp = W.generate("T256_H8_bf16_f32", lengths=[70, 0, 200, 5], H=2, K=16, seed=905)
    cu = inp.cu_seqlens
    X = oracle.kkt_solve_ref(inp.k64(), inp.g, inp.beta, cu, chunk_size=chunk)
    Wm = a_scale(inp.k64(), inp.g, inp.beta, cu, chunk)
    got = solve_bound(X, Wm, 3.0, cu)
    local, length = W.chunk_geometry(inp.workload.T, cu, chunk)
    rng = np.random.default_rng(906)
    for t in rng.integers(0, inp.workload.T, 12):
        h = int(rng.integers(0, 2))
        i, L, t0 = int(local[t]), int(length[t]), int(t - local[t])
        for j in range(chunk):
            want = 0.0
            if j < L:
                for m in range(L):
                    for n in range(L):
                        w = (1.0 if m == n else 0.0) + Wm[0, t0 + m, h, n]
                        want += abs(X[0, t0 + i, h, m]) * w * abs(X[0, t0 + n, h, j])
            assert got[0, t, h, j] == pytest.approx(3.0 * U32 * want, rel=1e-12, abs=1e-300)


def test_fp32_solve_meets_the_f16_bound():
    """With 128-token chunks and keys of few dimensions (24), a plain fp32
    computation of the rows rounded to f16 misses the one-ulp rule in a few
    elements (terms of a row cancel), stays far within the fp32 bound, and a
    planted error beyond the bound still fails."""
    inp = W.generate("T256_H8_bf16_f32", B=1, T=1024, H=4, K=24, in_dtype="f16", gate=True, beta=False, seed=1)
    X = oracle.kkt_solve_ref(inp.k64(), inp.g, inp.beta, None, chunk_size=128)
    y = oracle.round_to_f16_bits(_fp32_inverse(inp, 128).astype(np.float64))
    with pytest.raises(AssertionError, match="beyond 1 ulp"):
        compare(y, X, "f16")
    bound = fused_bound(inp, X, 128)
    stats = compare(y, X, "f16", None, "fp32 substitution", bound)
    assert stats["n_bound"] > 0 and stats["max_err_over_bound"] < 0.05
    b = bound()
    exp_bits = oracle.round_to_f16_bits(X)
    pos = tuple(np.argwhere((np.abs(X) > 1e-3) & (np.abs(X) < 1e-2))[0])
    bad = y.copy()
    moved = X[pos] + np.sign(X[pos]) * 2 * b[pos]
    bad[pos] = oracle.round_to_f16_bits(np.array(moved))
    assert abs(int(bad[pos]) - int(exp_bits[pos])) > 1
    with pytest.raises(AssertionError, match="beyond 1 ulp"):
        compare(bad, X, "f16", None, "planted", bound)
