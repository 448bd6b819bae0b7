"""GPU parity of the unfused two-step chain (MindSpeed-Ops PR #135, PR
description: the fused op stands for chunk_scaled_dot_kkt_fwd followed by
solve_tril): ``kkt_scaled_dot`` against the oracle's A, ``kkt_solve_tril``
against the oracle's solve of the same fp32 A, and the chain against the
fused entry point bit for bit.

Every case prints what it runs before touching the GPU.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from chunked_gated_delta_token_amd import workloads as W
from tests import _edge
from tests._compare import a_scale, compare, compare_A, structural_masks, tril_bound
from tests._gpu_util import TORCH_DT, from_device, load_kkt, say, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kkt():
    return load_kkt()


def describe(inp: W.Inputs, label: str) -> str:
    w = inp.workload
    return (f"[case] {label}: B={w.B} T={w.T} H={w.H} K={w.K} in={w.in_dtype} "
            f"g={inp.g is not None} beta={inp.beta is not None} "
            f"seqs={0 if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1}")


def gpu_scaled_dot(kkt, tensors) -> torch.Tensor:
    k, g, b, cu = tensors
    B, T, H, _ = k.shape
    A = torch.full((B, T, H, 64), float("nan"), dtype=torch.float32, device=k.device)
    kkt.kkt_scaled_dot(k, g, b, cu, out=A)
    torch.cuda.synchronize()
    return A


def gpu_solve_tril(kkt, A: torch.Tensor, cu, out_dtype: str) -> np.ndarray:
    B, T, H, _ = A.shape
    out = torch.full((B, T, H, 64), float("nan"), dtype=TORCH_DT[out_dtype], device=A.device)
    kkt.kkt_solve_tril(A, cu, output_dtype=TORCH_DT[out_dtype], out=out)
    torch.cuda.synchronize()
    return from_device(out, out_dtype)


def gpu_fused(kkt, tensors, out_dtype: str) -> np.ndarray:
    k, g, b, cu = tensors
    B, T, H, _ = k.shape
    out = torch.full((B, T, H, 64), float("nan"), dtype=TORCH_DT[out_dtype], device=k.device)
    kkt.kkt_solve(k, g, b, cu, output_dtype=TORCH_DT[out_dtype], out=out)
    torch.cuda.synchronize()
    return from_device(out, out_dtype)


def check_scaled_dot(kkt, inp: W.Inputs, label: str) -> dict:
    say(describe(inp, "scaled_dot " + label))
    got = gpu_scaled_dot(kkt, to_device(inp)).cpu().numpy()
    k64 = inp.k64()
    ref = oracle.scaled_dot_ref(k64, inp.g, inp.beta, inp.cu_seqlens)
    scale = a_scale(k64, inp.g, inp.beta, inp.cu_seqlens)
    stats = compare_A(got, ref, scale, inp.workload.K, inp.cu_seqlens, label)
    say("[ok] " + json.dumps(stats))
    return stats


def oracle_A_with_garbage(inp: W.Inputs, fill: float = float("nan")) -> np.ndarray:
    """The oracle's A rounded to fp32, with ``fill`` everywhere outside the
    strictly lower part of each chunk (the solve must not read it)."""
    A = oracle.scaled_dot_ref(inp.k64(), inp.g, inp.beta, inp.cu_seqlens).astype(np.float32)
    _d, _u, lower = structural_masks(inp.workload.T, inp.cu_seqlens)
    A[~np.broadcast_to(lower[None, :, None, :], A.shape)] = fill
    return A


def check_solve_tril(kkt, inp: W.Inputs, out_dtype: str, label: str) -> dict:
    say(describe(inp, f"solve_tril {label} out={out_dtype}"))
    A = oracle_A_with_garbage(inp)
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to("cuda:0")
    got = gpu_solve_tril(kkt, torch.from_numpy(A).to("cuda:0"), cu, out_dtype)
    ref = oracle.solve_tril_ref(A.astype(np.float64), inp.cu_seqlens)
    stats = compare(got, ref, out_dtype, inp.cu_seqlens, label, tril_bound(A, ref, inp.cu_seqlens))
    say("[ok] " + json.dumps(stats))
    return stats


def check_chain_equals_fused(kkt, inp: W.Inputs, out_dtype: str, label: str):
    say(describe(inp, f"chain == fused {label} out={out_dtype}"))
    t = to_device(inp)
    A = gpu_scaled_dot(kkt, t)
    chain = gpu_solve_tril(kkt, A, t[3], out_dtype)
    fused = gpu_fused(kkt, t, out_dtype)
    view = np.uint32 if out_dtype == "f32" else np.uint16
    diff = int(np.sum(chain.view(view) != fused.view(view)))
    assert diff == 0, f"{label}: {diff} elements differ between the chain and the fused op"
    say("[ok] bit-identical")


# ---------------------------------------------------------------- full workloads
@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_scaled_dot_full_parity(kkt, name):
    check_scaled_dot(kkt, W.generate(name), name)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_solve_tril_full_parity(kkt, name):
    inp = W.generate(name)
    check_solve_tril(kkt, inp, inp.workload.out_dtype, name)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_chain_equals_fused_full(kkt, name):
    inp = W.generate(name)
    check_chain_equals_fused(kkt, inp, inp.workload.out_dtype, name)


# ---------------------------------------------------------------- dtypes, head dims, shapes
@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("K", [32, 64, 96, 128, 224, 256])
def test_scaled_dot_dtypes_and_head_dims(kkt, in_dtype, K):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=150, H=3, K=K, in_dtype=in_dtype, seed=1100 + K)
    check_scaled_dot(kkt, inp, f"{in_dtype} K={K}")


def test_scaled_dot_fp32_keys_across_magnitudes(kkt):
    """Unnormalised fp32 keys scaled per token by 10^u, u uniform in
    [-15, 15]: the three-part bf16 split of fp32 keys keeps its relative
    accuracy at every magnitude (A is checked against a bound proportional to
    the magnitude of its own terms)."""
    inp = W.generate("T256_H8_bf16_f32", T=256, H=3, K=128, in_dtype="f32", seed=1150)
    rng = np.random.default_rng(1151)
    scale = 10.0 ** rng.uniform(-15.0, 15.0, inp.k_store.shape[:-1] + (1,))
    inp.k_store = (inp.k_store.astype(np.float64) * scale).astype(np.float32)
    check_scaled_dot(kkt, inp, "fp32 keys over 30 decades")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_solve_tril_out_dtypes(kkt, out_dtype):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=200, H=3, seed=1200)
    check_solve_tril(kkt, inp, out_dtype, "dtype")


@pytest.mark.parametrize("T", [1, 2, 17, 63, 64, 65, 129])
def test_split_lengths(kkt, T):
    gate, beta = bool(T % 2), bool((T // 2) % 2)
    inp = W.generate("T256_H8_bf16_f32", B=2, T=T, H=2, seed=1300 + T, gate=gate, beta=beta)
    check_scaled_dot(kkt, inp, f"T={T}")
    check_solve_tril(kkt, inp, "f32", f"T={T}")
    check_chain_equals_fused(kkt, inp, "f32", f"T={T}")


SPLIT_VARLEN = {
    "tiny_and_empty": [1, 2, 3, 0, 64, 65, 0, 130, 5],
    "many_short": [1, 3] * 70,
    "two_levels_1000": [0 if i % 6 == 0 else 1 + (i * 37) % 90 for i in range(1000)],
}


@pytest.mark.parametrize("case", list(SPLIT_VARLEN))
def test_split_varlen(kkt, case):
    lens = SPLIT_VARLEN[case]
    inp = W.generate("T256_H8_bf16_f32", lengths=lens, H=3, seed=1400)
    check_scaled_dot(kkt, inp, f"varlen {case}")
    check_solve_tril(kkt, inp, "f32", f"varlen {case}")
    check_chain_equals_fused(kkt, inp, "bf16", f"varlen {case}")


@pytest.mark.parametrize("in_dtype,out_dtype", [("f32", "f16"), ("f16", "bf16"), ("bf16", "f32")])
def test_chain_equals_fused_dtypes(kkt, in_dtype, out_dtype):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=300, H=3, K=256 if in_dtype == "f16" else 128,
                     in_dtype=in_dtype, seed=1500)
    check_chain_equals_fused(kkt, inp, out_dtype, f"{in_dtype}->{out_dtype}")


def test_split_large_gate_spread(kkt):
    """Gate differences beyond +-50 inside a chunk: both halves take the
    clamped path, and the chain still equals the fused op."""
    inp = W.generate("T256_H8_bf16_f32", T=128, H=2, seed=1600)
    rng = np.random.default_rng(1601)
    inc = -rng.uniform(0.0, 3.0, inp.g.shape)
    g = np.empty_like(inc)
    for t0 in range(0, 128, 64):
        g[:, t0:t0 + 64] = np.cumsum(inc[:, t0:t0 + 64], axis=1)
    inp.g = g.astype(np.float32)
    check_scaled_dot(kkt, inp, "gate spread ~ -96")
    check_solve_tril(kkt, inp, "f32", "gate spread ~ -96")
    check_chain_equals_fused(kkt, inp, "f32", "gate spread ~ -96")


# ---------------------------------------------------------------- properties of the solve alone
def test_solve_tril_reads_only_the_strict_lower_part(kkt):
    """NaN, zeros or random values outside the strictly lower part of A give
    bit-identical results."""
    inp = W.generate("T256_H8_bf16_f32", T=190, H=3, seed=1700)
    say(describe(inp, "solve_tril ignores diagonal and upper part"))
    outs = []
    rng = np.random.default_rng(1701)
    for fill in (float("nan"), 0.0, None):
        A = oracle_A_with_garbage(inp, 0.0 if fill is None else fill)
        if fill is None:
            _d, _u, lower = structural_masks(inp.workload.T)
            noise = rng.standard_normal(A.shape).astype(np.float32)
            A = np.where(np.broadcast_to(lower[None, :, None, :], A.shape), A, noise)
        outs.append(gpu_solve_tril(kkt, torch.from_numpy(np.ascontiguousarray(A)).to("cuda:0"), None, "f32"))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_solve_tril_of_zero_is_identity(kkt):
    T, H = 130, 2
    say(f"[case] solve_tril of A = 0: T={T} H={H}")
    A = torch.zeros((1, T, H, 64), dtype=torch.float32, device="cuda:0")
    got = gpu_solve_tril(kkt, A, None, "f32")
    local, length = W.chunk_geometry(T)
    exp = np.zeros((1, T, H, 64), dtype=np.float32)
    exp[0, np.arange(T), :, local] = 1.0
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))


# ---------------------------------------------------------------- hand-worked values on the GPU
def test_hand_worked_golden_split(kkt):
    """The worked chunks: A from kkt_scaled_dot against the hand-derived a_ij,
    and the solve of those hand values against the hand-derived inverse."""
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_chunks.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        say(f"[case] golden split {c['name']}")
        kk = np.array(c["k"], dtype=np.float64)
        T, Kc = kk.shape
        k = np.zeros((1, T, 1, 64), dtype=np.float32)
        k[0, :, 0, :Kc] = kk           # zero padding keeps every dot product
        wl = W.Workload("golden", 1, T, 1, 64, "f32", "f32", c["g"] is not None, c["beta"] is not None, 0)
        inp = W.Inputs(wl, k,
                       None if c["g"] is None else np.array(c["g"], dtype=np.float32).reshape(1, T, 1),
                       None if c["beta"] is None else np.array(c["beta"], dtype=np.float32).reshape(1, T, 1),
                       None if c["cu_seqlens"] is None else np.array(c["cu_seqlens"], dtype=np.int32))
        t = to_device(inp)
        A = gpu_scaled_dot(kkt, t)
        got_A = A.cpu().numpy()
        hand_A = np.zeros((1, T, 1, 64), dtype=np.float32)
        for i, row in enumerate(c["expected_A_rows"]):
            hand_A[0, i, 0, :len(row)] = row
        # relative 1e-5: fp32 exp of gate differences up to 50 (see the fused golden test)
        tol = 1e-5 * np.maximum(np.abs(hand_A.astype(np.float64)), 1e-30)
        assert np.all(np.abs(got_A - hand_A) <= tol), (c["name"], got_A[0, :, 0, :T])
        cu = t[3]
        got = gpu_solve_tril(kkt, torch.from_numpy(hand_A).to("cuda:0"), cu, "f32")
        for i, row in enumerate(c["expected_rows"]):
            exp = np.zeros(64)
            exp[:len(row)] = row
            assert np.all(np.abs(got[0, i, 0] - exp) <= 1e-6 * np.maximum(np.abs(exp), 1.0)), (c["name"], i)


@pytest.mark.parametrize("kind", _edge.KINDS)
def test_edge_inputs_unfused_chain(kkt, kind):
    """The edge inputs through the two unfused steps: A against the oracle,
    the solve of the oracle's A, and the chain bit-equal to the fused op."""
    inp = _edge.edge_inputs(kind, 2400, 8, seed=690)
    check_scaled_dot(kkt, inp, kind)
    check_solve_tril(kkt, inp, "f32", kind)
    check_chain_equals_fused(kkt, inp, "f32", kind)
