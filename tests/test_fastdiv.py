"""The launch-constant division the kernels use for tile -> (chunk, head) and
chunk -> (batch row, chunk): mulhi(n, magic) >> shift with the host's
(magic, shift) for d, or n >> shift for a power of two.  Restated here from
its definition (the comment at FastDiv in the kernel source) and checked
against integer division: every divisor up to 4096 on dividends around each
multiple of d, random dividends below 2^31, and divisors near 2^31."""
from __future__ import annotations

import numpy as np


def make_fastdiv(d: int):
    s = d.bit_length() - 1          # floor(log2 d)
    if 1 << s == d:
        return 0, s
    magic = ((1 << (32 + s)) + d - 1) // d
    assert (1 << 31) < magic < (1 << 32)
    return magic, s


def fast_div(n, magic, shift):
    n = np.asarray(n, dtype=np.uint64)
    if magic == 0:
        return n >> np.uint64(shift)
    return ((n * np.uint64(magic)) >> np.uint64(32)) >> np.uint64(shift)


def test_small_divisors_exhaustive_near_multiples():
    top = (1 << 31) - 1
    for d in range(1, 4097):
        magic, shift = make_fastdiv(d)
        q = np.arange(0, top // d + 1, max(1, (top // d) // 2000), dtype=np.uint64)
        n = np.concatenate([q * d, q * d + (d - 1), q * d - 1, [top, top - 1]])
        n = n[(n >= 0) & (n <= top)].astype(np.uint64)
        assert np.array_equal(fast_div(n, magic, shift), n // np.uint64(d)), d


def test_random_and_large_divisors():
    rng = np.random.default_rng(7)
    n = rng.integers(0, 1 << 31, size=200_000, dtype=np.uint64)
    for d in list(rng.integers(2, 1 << 31, size=300)) + [(1 << 31) - 1, (1 << 30) + 1, 3 << 29, 65537, 96 * 257]:
        d = int(d)
        magic, shift = make_fastdiv(d)
        assert np.array_equal(fast_div(n, magic, shift), n // np.uint64(d)), d
