"""Tensors past 4 GiB: (1, 2359296, 8, 128) bf16 keys are 4.5 GiB, so the
tiles from token 2097152 on start beyond byte 2^32 of k (and of an fp32
64-wide or bf16 128-wide output).  The inputs are drawn on the GPU from a
seeded torch generator (host generation in fp64 would need about 19 GB);
the oracle checks sampled chunks at the start, on both sides of the 2^32
boundary and at the end, by the criteria of the other parity tests.

Every case prints what it runs before touching the GPU.
"""
from __future__ import annotations

import json

import numpy as np
import pytest

import oracle
from tests._compare import compare
from tests._gpu_util import load_kkt, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

T, H, K = 2359296, 8, 128            # 36864 chunks of 64 tokens
BOUNDARY = (1 << 32) // (H * K * 2)  # first token whose key row starts at byte 2^32


@pytest.fixture(scope="module")
def kkt():
    return load_kkt()


@pytest.fixture(scope="module")
def big_inputs(kkt):
    """k: rows of N(0,1)/sqrt(K) rounded to bf16; beta = sigmoid(N(0,1));
    g: running sum of logsigmoid(N(4,1)) restarted every 64 tokens (whole
    128-token chunks then see two restarts, which the formula allows)."""
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(7100)
    dev = torch.device("cuda:0")
    say(f"[case] large offsets: generating (1, {T}, {H}, {K}) bf16 keys on the GPU")
    k = torch.empty((1, T, H, K), dtype=torch.bfloat16, device=dev)
    step = 1 << 18
    for t0 in range(0, T, step):  # in slabs, to bound the fp32 temporary
        n = min(step, T - t0)
        k[:, t0:t0 + n] = (torch.randn((1, n, H, K), generator=gen, device=dev) / np.sqrt(K)).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((1, T, H), generator=gen, device=dev))
    a = torch.nn.functional.logsigmoid(torch.randn((1, T, H), generator=gen, device=dev) + 4.0)
    g = a.view(1, T // 64, 64, H).cumsum(dim=2).view(1, T, H).contiguous()
    torch.cuda.synchronize()
    return k, g, beta


def _sampled_chunks(chunk):
    last = T // chunk - 1
    b = BOUNDARY // chunk
    return sorted({0, b - 1, b, b + 1, last})


def _oracle_chunk(k, g, beta, t0, chunk, h):
    kk = k[:, t0:t0 + chunk, h:h + 1].float().cpu().numpy().astype(np.float64)
    gg = g[:, t0:t0 + chunk, h:h + 1].cpu().numpy()
    bb = beta[:, t0:t0 + chunk, h:h + 1].cpu().numpy()
    return oracle.kkt_solve_ref(kk, gg, bb, None, chunk_size=chunk)


@pytest.mark.parametrize("chunk,out_dtype", [(64, "f32"), (128, "bf16")])
def test_tiles_beyond_4gib(kkt, big_inputs, chunk, out_dtype):
    k, g, beta = big_inputs
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    say(f"[case] large offsets: kkt_solve chunk={chunk} out={out_dtype}, output "
        f"{T * H * chunk * tdt.itemsize / 2**30:.2f} GiB")
    out = torch.full((1, T, H, chunk), float("nan"), dtype=tdt, device=k.device)
    kkt.kkt_solve(k, g, beta, chunk_size=chunk, output_dtype=tdt, out=out)
    torch.cuda.synchronize()
    assert BOUNDARY * H * K * 2 == 1 << 32 and BOUNDARY < T
    for c in _sampled_chunks(chunk):
        t0 = c * chunk
        for h in (0, H - 1):
            ref = _oracle_chunk(k, g, beta, t0, chunk, h)
            o = out[:, t0:t0 + chunk, h:h + 1]
            got = o.cpu().numpy() if out_dtype == "f32" else o.view(torch.int16).cpu().numpy().view(np.uint16)
            stats = compare(got, ref, out_dtype, None, f"chunk {c} head {h}")
            say("[ok] " + json.dumps(stats))
    # no element is left unwritten anywhere
    assert not torch.isnan(out.float() if out_dtype != "f32" else out).any().item()
