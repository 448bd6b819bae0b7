"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from chunked_gated_delta_token_amd import workloads
from tests import oracle_pins


def _solve(k, g, beta, cu, **kw):
    return oracle.kkt_solve_ref(k, g, beta, cu, **kw)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(_solve)


@pytest.mark.parametrize("pin", oracle_pins.SPLIT_PINS, ids=lambda f: f.__name__)
def test_split_pin(pin):
    pin(_solve, lambda k, g, b, cu: oracle.scaled_dot_ref(k, g, b, cu),
        lambda A, cu=None: oracle.solve_tril_ref(A, cu))


@pytest.mark.parametrize("pin", oracle_pins.CHUNK128_PINS, ids=lambda f: f.__name__)
def test_chunk128_pin(pin):
    pin(_solve)


@pytest.mark.parametrize("pin", oracle_pins.CUMSUM_PINS, ids=lambda f: f.__name__)
def test_cumsum_pin(pin):
    pin(_solve, lambda a, cu=None, chunk=64: oracle.chunk_cumsum_ref(a, cu, chunk))


@pytest.mark.parametrize("name", ["T2000_H8_bf16_bf16"])
def test_cumsum_agrees_with_the_input_recipe(name):
    """The recipe's gate (summed in fp64, then rounded to fp32) and the
    oracle's chunk-local sum of the recipe's fp32 decays agree to the fp32
    rounding of both; packed sequences restart the sum too."""
    for lengths in (None, [70, 1, 0, 129, 300]):
        inp = workloads.generate(name, T=None if lengths else 300, H=3, lengths=lengths)
        g = oracle.chunk_cumsum_ref(inp.g_raw, inp.cu_seqlens)
        prefix_abs = oracle.chunk_cumsum_ref(np.abs(inp.g_raw.astype(np.float64)), inp.cu_seqlens)
        assert np.all(np.abs(g - inp.g) <= 2.0 ** -23 * (np.abs(g) + prefix_abs) + 1e-30)


def test_clamp_flag_is_the_pure_definition_when_off():
    # with the clamp off, a gate difference of 60 is exp(60)
    k = np.ones((1, 2, 1, 1))
    out = oracle.kkt_solve_ref(k, np.array([[[-60.0], [0.0]]]), None, None, clamp_gate=False)
    assert abs(out[0, 1, 0, 0] + np.exp(60.0)) <= 1e-9 * np.exp(60.0)


def test_rejects_bad_varlen():
    k = np.zeros((1, 5, 1, 4))
    with pytest.raises(ValueError):
        oracle.kkt_solve_ref(k, cu_seqlens=np.array([0, 3, 4], dtype=np.int32))  # does not end at T
    with pytest.raises(ValueError):
        oracle.kkt_solve_ref(k, cu_seqlens=np.array([0, 4, 3, 5], dtype=np.int32))  # decreasing


def test_chunk_size_is_a_parameter():
    # chunk 128 = a 128-token chunk; with orthogonal keys every chunk is I
    T = 128
    k = np.zeros((1, T, 1, T))
    k[0, np.arange(T), 0, np.arange(T)] = 1.0
    out = oracle.kkt_solve_ref(k, chunk_size=128)
    assert out.shape == (1, T, 1, 128) and np.array_equal(out[0, :, 0], np.eye(T))


# ---- expected value of a rounded output --------------------------------------
def _bf16_from_f32_bits_rne(x32):
    """Textbook integer round-to-nearest-even of fp32 bit patterns to bf16."""
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_rounding_matches_integer_rne_on_fp32_values():
    rng = np.random.default_rng(30)
    x32 = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 30, 200000))).astype(np.float32)
    assert np.array_equal(oracle.round_to_bf16_bits(x32.astype(np.float64)), _bf16_from_f32_bits_rne(x32))


def test_bf16_rounding_ties_and_no_double_rounding():
    # consecutive bf16 values a < b, their midpoint m: ties go to the even one;
    # m plus a hair (not an fp32 value) goes up, m minus a hair goes down
    bits = np.arange(0x3F80, 0x4000, dtype=np.uint16)   # [1, 2)
    a = workloads.bf16_bits_to_f64(bits[:-1])
    b = workloads.bf16_bits_to_f64(bits[1:])
    m = (a + b) / 2.0
    even = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(oracle.round_to_bf16_bits(m), even)
    hair = np.exp2(-40.0)
    assert np.array_equal(oracle.round_to_bf16_bits(m + hair), bits[1:])
    assert np.array_equal(oracle.round_to_bf16_bits(m - hair), bits[:-1])
    assert np.array_equal(oracle.round_to_bf16_bits(-(m + hair)), bits[1:] | 0x8000)


def test_bf16_rounding_agrees_with_the_input_cast():
    # two independent implementations (oracle output rounding, input cast)
    rng = np.random.default_rng(31)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-60, 60, 100000))
    assert np.array_equal(oracle.round_to_bf16_bits(x), workloads.f64_to_bf16_bits(x))


def test_f16_rounding_ties():
    one = 1.0
    ulp = 2.0 ** -10
    assert oracle.round_to_f16_bits(np.array([one + ulp / 2]))[0] == 0x3C00          # tie -> even (1.0)
    assert oracle.round_to_f16_bits(np.array([one + ulp / 2 + 2.0 ** -40]))[0] == 0x3C01
    assert oracle.round_to_f16_bits(np.array([one + 1.5 * ulp]))[0] == 0x3C02        # tie -> even
