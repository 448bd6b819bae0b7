"""Inputs outside the workloads' distributions that the formula still
defines (test infrastructure, no GPU): signed and zero beta, gates that rise
or wander instead of decaying, all-zero key rows and a whole zero chunk.
Each is sized so that the inverse stays moderate (max |X| below about 10 at
64-token chunks, 60 at 128), where the fp32 bars apply as stated."""
from __future__ import annotations

import numpy as np

from chunked_gated_delta_token_amd import workloads as W

KINDS = ("signed_beta", "rising_gate", "wandering_gate", "zero_keys")


def _gate(inp: W.Inputs, rng, lo: float, hi: float, chunk: int) -> None:
    """g = running sum of per-token steps in [lo, hi), restarted every chunk."""
    inc = rng.uniform(lo, hi, inp.g.shape)
    g = np.empty_like(inc)
    for t0 in range(0, inc.shape[1], chunk):
        g[:, t0:t0 + chunk] = np.cumsum(inc[:, t0:t0 + chunk], axis=1)
    inp.g = g.astype(np.float32)


def edge_inputs(kind: str, T: int, H: int, seed: int, chunk: int = 64) -> W.Inputs:
    inp = W.generate("T256_H8_bf16_f32", T=T, H=H, seed=seed)
    rng = np.random.default_rng(seed + 1)
    if kind == "signed_beta":
        b = rng.uniform(-1.5, 1.5, inp.beta.shape)
        b[rng.random(b.shape) < 0.1] = 0.0
        inp.beta = b.astype(np.float32)
    elif kind == "rising_gate":
        _gate(inp, rng, 0.0, 0.1 if chunk == 64 else 0.05, chunk)
    elif kind == "wandering_gate":
        _gate(inp, rng, -0.3, 0.3, chunk)
    elif kind == "zero_keys":
        ks = inp.k_store.copy()
        ks[:, rng.random(T) < 0.2] = 0          # +0.0 in every key dtype
        ks[:, 128:256] = 0                       # whole chunks of zero keys
        inp.k_store = ks
    else:
        raise ValueError(kind)
    return inp
