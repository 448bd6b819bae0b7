"""The acceptance criteria of the GPU tests, exercised on the CPU: the
oracle's own results rounded as a kernel would round them pass, and the
mistakes the criteria exist for (an unwritten element, a nonzero where the
output must be +0.0, an error beyond the bound) fail."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from chunked_gated_delta_token_amd import workloads as W
from tests._compare import GATE_ULPS, U32, a_scale, compare, compare_A


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
