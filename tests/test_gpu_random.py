"""Seeded random configurations against the oracle.

Sizes, head counts and dimensions, key and output dtypes, gate and beta
presence, packed sequences (empty ones among them), chunk sizes and entry
points are drawn from fixed seeds, so every run checks the same cases: 96
with K in {64, 128, 256}, then 48 with any K the library serves (up to 256,
fp32 keys a multiple of 4, 16-bit keys a multiple of 8).  Each is small
enough for the oracle to finish at once.  The criteria are those of the
targeted tests (their check functions are reused).
"""
from __future__ import annotations

import numpy as np
import pytest

from chunked_gated_delta_token_amd import workloads as W
from tests import test_gpu_chunk128 as c128
from tests import test_gpu_gate_cumsum as gc
from tests import test_gpu_parity as fused
from tests import test_gpu_split as split
from tests._gpu_util import load_kkt

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ENTRIES = ("fused", "fused128", "gate_cumsum", "chain")
DTYPES = ("bf16", "f16", "f32")


def _draw_cases(n=96, seed=9000, any_k=False, first=0):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        entry = ENTRIES[i % len(ENTRIES)]
        c = dict(entry=entry, H=int(rng.integers(1, 10)), K=int(rng.choice([64, 128, 256])),
                 in_dtype=str(rng.choice(DTYPES)), out_dtype=str(rng.choice(DTYPES)),
                 gate=bool(rng.random() < 0.75) or entry == "gate_cumsum", beta=bool(rng.random() < 0.75),
                 seed=9100 + first + i)
        if any_k:
            # rows of whole 16-byte pieces: multiples of 4 (fp32) or 8 (16-bit)
            step = 4 if c["in_dtype"] == "f32" else 8
            c["K"] = int(rng.integers(1, 256 // step + 1)) * step
        if rng.random() < 0.4:
            n_seqs = int(rng.integers(1, 90))
            lens = rng.integers(0, 300, size=n_seqs)
            lens[rng.random(n_seqs) < 0.15] = 0
            if lens.sum() == 0:
                lens[0] = 1
            c["lengths"] = [int(x) for x in lens]
        else:
            c["B"] = int(rng.integers(1, 4))
            c["T"] = int(rng.integers(1, 700))
        cases.append(c)
    return cases


CASES = _draw_cases() + _draw_cases(n=48, seed=9500, any_k=True, first=96)


@pytest.fixture(scope="module")
def kkt():
    return load_kkt()


def _label(i, c):
    shape = f"seqs={len(c['lengths'])}" if "lengths" in c else f"B={c['B']} T={c['T']}"
    return (f"random {i} {c['entry']} {shape} H={c['H']} K={c['K']} {c['in_dtype']}->{c['out_dtype']} "
            f"g={c['gate']} beta={c['beta']}")


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_configuration(kkt, i):
    c = CASES[i]
    over = {k: c[k] for k in ("H", "K", "in_dtype", "gate", "beta", "seed")}
    if "lengths" in c:
        over["lengths"] = c["lengths"]
    else:
        over["B"], over["T"] = c["B"], c["T"]
    inp = W.generate("T256_H8_bf16_f32", **over)
    label = _label(i, c)
    if c["entry"] == "fused":
        fused.check(kkt, inp, c["out_dtype"], label)
    elif c["entry"] == "fused128":
        c128.check(kkt, inp, c["out_dtype"], label)
    elif c["entry"] == "gate_cumsum":
        gc.check(kkt, inp, c["out_dtype"], label)
    else:
        split.check_scaled_dot(kkt, inp, label)
        split.check_chain_equals_fused(kkt, inp, c["out_dtype"], label)
