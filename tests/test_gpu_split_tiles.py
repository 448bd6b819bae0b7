"""GPU: the fused op's two launch forms give the same bits.

Small grids run each 64-token tile on a two-wave workgroup (the first wave
finishes block rows 0..2, the second block row 3, exchanging the diagonal
inverses and X10, X21, X20 through LDS); large grids run one tile per wave.
Both form every block by the same operations in the same order, so their
outputs must be bit-identical.  The library option KKT_OPTION_SPLIT_MAX_TILES
forces one form or the other on the same inputs; each case is also checked
against the fp64 oracle.
"""
from __future__ import annotations

import json

import numpy as np
import pytest

import oracle
from chunked_gated_delta_token_amd import workloads as W
from tests._compare import compare, fused_bound
from tests._gpu_util import TORCH_DT, from_device, load_kkt, say, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SPLIT_ALL = 1_000_000_000  # a two-wave bound above every grid here


@pytest.fixture(scope="module")
def kkt():
    return load_kkt()


def run_form(kkt, t, out_dtype: str, split: bool) -> np.ndarray:
    k, g, b, cu = t
    B, T, H, _ = k.shape
    with kkt.option(kkt.KKT_OPTION_SPLIT_MAX_TILES, SPLIT_ALL if split else 0):
        out = torch.full((B, T, H, 64), float("nan"), dtype=TORCH_DT[out_dtype], device=k.device)
        kkt.kkt_solve(k, g, b, cu, output_dtype=TORCH_DT[out_dtype], out=out)
        torch.cuda.synchronize()
    return from_device(out, out_dtype)


def both_forms(kkt, inp: W.Inputs, out_dtype: str, label: str):
    w = inp.workload
    say(f"[case] split vs one-wave tiles, {label}: B={w.B} T={w.T} H={w.H} K={w.K} in={w.in_dtype} "
        f"out={out_dtype} g={inp.g is not None} beta={inp.beta is not None} "
        f"seqs={0 if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1}")
    t = to_device(inp)
    one = run_form(kkt, t, out_dtype, split=False)
    two = run_form(kkt, t, out_dtype, split=True)
    view = np.uint32 if out_dtype == "f32" else np.uint16
    assert np.array_equal(one.view(view), two.view(view)), label
    ref = oracle.kkt_solve_ref(inp.k64(), inp.g, inp.beta, inp.cu_seqlens)
    stats = compare(two, ref, out_dtype, inp.cu_seqlens, label, fused_bound(inp, ref))
    say("[ok] " + json.dumps(stats))


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_split_tiles_workloads(kkt, name):
    """Every workload at full size (the large one included, forced split)."""
    inp = W.generate(name)
    both_forms(kkt, inp, inp.workload.out_dtype, name)


@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [64, 256])
def test_split_tiles_dtypes_and_K(kkt, in_dtype, out_dtype, K):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=333, H=3, K=K, in_dtype=in_dtype, seed=4100 + K)
    both_forms(kkt, inp, out_dtype, f"{in_dtype}->{out_dtype} K={K}")


@pytest.mark.parametrize("gate,beta", [(False, False), (True, False), (False, True)])
def test_split_tiles_without_gate_or_beta(kkt, gate, beta):
    inp = W.generate("T256_H8_bf16_f32", B=1, T=1000, H=5, seed=4200, gate=gate, beta=beta)
    both_forms(kkt, inp, "f32", f"gate={gate} beta={beta}")


@pytest.mark.parametrize("T", [1, 2, 17, 48, 63, 64, 65, 130])
def test_split_tiles_short_chunks(kkt, T):
    """Partial chunks: one or both waves' rows past the chunk's end."""
    inp = W.generate("T256_H8_bf16_f32", B=3, T=T, H=2, seed=4300 + T)
    both_forms(kkt, inp, "f32", f"T={T}")


def test_split_tiles_gate_beyond_clamp(kkt):
    """Within-chunk gate differences beyond +-50: the clamped per-element
    epilogue instead of the factored one."""
    inp = W.generate("T256_H8_bf16_f32", T=256, H=4, seed=4400)
    rng = np.random.default_rng(4401)
    inc = -rng.uniform(0.0, 3.0, inp.g.shape)
    g = np.empty_like(inc)
    for t0 in range(0, 256, 64):
        g[:, t0:t0 + 64] = np.cumsum(inc[:, t0:t0 + 64], axis=1)
    inp.g = g.astype(np.float32)
    both_forms(kkt, inp, "f32", "gate spread ~ -96")


def test_split_tiles_packed_short_sequences(kkt):
    """Packed sequences with empty and one-token members."""
    lens = np.random.default_rng(4500).integers(0, 150, 40)
    lens[[3, 17]] = 0
    lens[[5, 30]] = 1
    inp = W.generate("T256_H8_bf16_f32", lengths=lens.tolist(), H=3, seed=4501)
    both_forms(kkt, inp, "f32", "packed 40 short sequences")


def run_gate_sum_form(kkt, inp: W.Inputs, split: bool, in_place: bool):
    k, _, b, cu = to_device(inp)
    g_raw = torch.from_numpy(inp.g_raw).to(k.device)
    with kkt.option(kkt.KKT_OPTION_SPLIT_MAX_TILES, SPLIT_ALL if split else 0):
        B, T, H, _ = k.shape
        out = torch.full((B, T, H, 64), float("nan"), dtype=torch.float32, device=k.device)
        g_out = g_raw if in_place else torch.full((B, T, H), float("nan"), dtype=torch.float32, device=k.device)
        kkt.kkt_solve_gate_cumsum(k, g_raw, b, cu, output_dtype=torch.float32, out=out, g_out=g_out)
        torch.cuda.synchronize()
    return out.cpu().numpy(), g_out.cpu().numpy()


@pytest.mark.parametrize("shape", ["T256", "T2000", "packed"])
def test_split_tiles_gate_sum(kkt, shape):
    """kkt_solve_gate_cumsum: the two forms give the same bits for the output
    and the summed gate, also summing in place (g_out = g_decay, which the
    second wave of a split tile reads while the first one writes the sums)."""
    if shape == "packed":
        lens = np.random.default_rng(4600).integers(0, 300, 30)
        lens[[2, 9]] = 0
        inp = W.generate("T256_H8_bf16_f32", lengths=lens.tolist(), H=3, seed=4601)
    else:
        inp = W.generate("T2000_H8_bf16_bf16" if shape == "T2000" else "T256_H8_bf16_f32")
    say(f"[case] gate-sum split vs one-wave tiles, {shape}: B={inp.workload.B} T={inp.workload.T} H={inp.workload.H}")
    X1, g1 = run_gate_sum_form(kkt, inp, split=False, in_place=False)
    X2, g2 = run_gate_sum_form(kkt, inp, split=True, in_place=False)
    X3, g3 = run_gate_sum_form(kkt, inp, split=True, in_place=True)
    for X in (X2, X3):
        assert np.array_equal(X1.view(np.uint32), X.view(np.uint32))
    if inp.cu_seqlens is None:
        for g in (g2, g3):
            assert np.array_equal(g1.view(np.uint32), g.view(np.uint32))
    else:
        covered = np.zeros(inp.workload.T, dtype=bool)
        covered[int(inp.cu_seqlens[0]):int(inp.cu_seqlens[-1])] = True
        for g in (g2, g3):
            assert np.array_equal(g1[:, covered].view(np.uint32), g[:, covered].view(np.uint32))
    ref = oracle.kkt_solve_ref(inp.k64(), inp.g, inp.beta, inp.cu_seqlens)
    compare(X3, ref, "f32", inp.cu_seqlens, f"gate-sum split {shape}")
    say("[ok]")


def test_split_tiles_many_packed_sequences(kkt):
    """More than 64 packed sequences (the 64-ary chunk search instead of the
    scan) on a grid small enough for two-wave tiles."""
    lens = np.random.default_rng(4700).integers(0, 12, 110)
    lens[[0, 50, 109]] = 0
    inp = W.generate("T256_H8_bf16_f32", lengths=lens.tolist(), H=2, seed=4701)
    assert 2 * (inp.workload.T // 64 + 110) <= 256
    both_forms(kkt, inp, "f32", "packed 110 short sequences")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", ["T2000", "packed"])
def test_split_tiles_solve_tril(kkt, shape, out_dtype):
    """kkt_solve_tril of the same A in both forms: the same bits, and the
    chain kkt_solve_tril(kkt_scaled_dot(...)) bit-equal to the fused op."""
    if shape == "packed":
        lens = np.random.default_rng(4800).integers(0, 200, 25)
        lens[[1, 7]] = 0
        inp = W.generate("T256_H8_bf16_f32", lengths=lens.tolist(), H=3, seed=4801)
    else:
        inp = W.generate("T2000_H8_bf16_bf16")
    say(f"[case] solve_tril split vs one-wave tiles, {shape} -> {out_dtype}")
    k, g, b, cu = to_device(inp)
    A = kkt.kkt_scaled_dot(k, g, b, cu)
    torch.cuda.synchronize()
    res = []
    for split in (False, True):
        with kkt.option(kkt.KKT_OPTION_SPLIT_MAX_TILES, SPLIT_ALL if split else 0):
            X = kkt.kkt_solve_tril(A, cu, output_dtype=TORCH_DT[out_dtype])
            torch.cuda.synchronize()
        res.append(from_device(X, out_dtype))
    view = np.uint32 if out_dtype == "f32" else np.uint16
    assert np.array_equal(res[0].view(view), res[1].view(view))
    fused = run_form(kkt, (k, g, b, cu), out_dtype, split=True)
    assert np.array_equal(res[1].view(view), fused.view(view))
    ref = oracle.kkt_solve_ref(inp.k64(), inp.g, inp.beta, inp.cu_seqlens)
    compare(res[1], ref, out_dtype, inp.cu_seqlens, f"solve_tril split {shape}", fused_bound(inp, ref))
    say("[ok]")
