"""GPU parity of ``kkt_solve_gate_cumsum``: the fused op fed with per-token
log-decays, the chunk-local sum formed in the kernel (64- and 128-token
chunks; with 128, the second half's 6-level scan is added to the first
half's total, 7 levels, still within the bound below).

Against the oracle: the summed gate within 8 2^-24 of the running sum of
|decay| (a 6-level fp32 tree sum has first-order error at most 6 2^-24 times
that sum; 8 leaves room for the higher-order terms), and the output rows by
the criteria of the fused op.  Against the library itself: ``kkt_solve`` on
the gate this call wrote gives bit-identical rows.
"""
from __future__ import annotations

import json

import numpy as np
import pytest

import oracle
from chunked_gated_delta_token_amd import workloads as W
from tests._compare import GATE_BOUND_ULPS, compare, fused_bound
from tests._gpu_util import TORCH_DT, from_device, load_kkt, say, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module")
def kkt():
    return load_kkt()


def run(kkt, inp: W.Inputs, out_dtype: str, with_gate_out=True, in_place=False, chunk=64):
    k, _g, b, cu = to_device(inp)
    a = torch.from_numpy(inp.g_raw).to(k.device)
    B, T, H, _ = k.shape
    out = torch.full((B, T, H, chunk), float("nan"), dtype=TORCH_DT[out_dtype], device=k.device)
    g_out = None
    if in_place:
        g_out = a
    elif with_gate_out:
        g_out = torch.full((B, T, H), float("nan"), dtype=torch.float32, device=k.device)
    kkt.kkt_solve_gate_cumsum(k, a, b, cu, chunk_size=chunk, output_dtype=TORCH_DT[out_dtype], out=out, g_out=g_out)
    torch.cuda.synchronize()
    return from_device(out, out_dtype), (None if g_out is None else g_out.cpu().numpy())


def check(kkt, inp: W.Inputs, out_dtype: str, label: str, chunk: int = 64):
    w = inp.workload
    say(f"[case] gate_cumsum {label}: chunk={chunk} B={w.B} T={w.T} H={w.H} K={w.K} in={w.in_dtype} out={out_dtype} "
        f"beta={inp.beta is not None} seqs={0 if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1}")
    got, g = run(kkt, inp, out_dtype, chunk=chunk)
    X_ref, g_ref = oracle.kkt_solve_gate_cumsum_ref(inp.k64(), inp.g_raw, inp.beta, inp.cu_seqlens, chunk_size=chunk)
    prefix_abs = oracle.chunk_cumsum_ref(np.abs(inp.g_raw.astype(np.float64)), inp.cu_seqlens, chunk_size=chunk)
    err = np.abs(g.astype(np.float64) - g_ref)
    bound = GATE_BOUND_ULPS * 2.0 ** -24 * prefix_abs
    assert not np.any(np.isnan(g)), f"{label}: unwritten gate rows"
    assert np.all(err <= bound), f"{label}: gate sum error {float(np.max(err / np.maximum(bound, 1e-300))):.2f} x bound"
    # the summed gate's error (checked above) enters every g_i - g_j twice
    gate_err = 2 * GATE_BOUND_ULPS * float(prefix_abs.max(initial=0.0))
    stats = compare(got, X_ref, out_dtype, inp.cu_seqlens, label, fused_bound(inp, X_ref, chunk, gate_err))
    stats["gate_err_over_bound"] = float(np.max(err / np.maximum(bound, 1e-300)))
    say("[ok] " + json.dumps(stats))
    # the same gate through kkt_solve gives the same rows, bit for bit
    k, _g, b, cu = to_device(inp)
    B, T, H, _ = k.shape
    out2 = torch.full((B, T, H, chunk), float("nan"), dtype=TORCH_DT[out_dtype], device=k.device)
    kkt.kkt_solve(k, torch.from_numpy(g).to(k.device), b, cu, chunk_size=chunk, output_dtype=TORCH_DT[out_dtype],
                  out=out2)
    torch.cuda.synchronize()
    view = np.uint32 if out_dtype == "f32" else np.uint16
    assert np.array_equal(from_device(out2, out_dtype).view(view), got.view(view)), f"{label}: kkt_solve differs"


GATED = [n for n, w in W.WORKLOADS.items() if w.gate]


@pytest.mark.parametrize("name", GATED)
def test_gate_cumsum_full_parity(kkt, name):
    inp = W.generate(name)
    check(kkt, inp, inp.workload.out_dtype, name)


def test_gate_cumsum_varlen_workload_with_gate(kkt):
    """The packed 12-sequence workload, drawn with a gate and beta."""
    inp = W.generate("varlen12_T16384_H7_f32_f32", gate=True, beta=True)
    check(kkt, inp, "f32", "varlen12 gated")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 129])
def test_gate_cumsum_lengths(kkt, T):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=T, H=3, seed=2000 + T, beta=bool(T % 2))
    check(kkt, inp, "f32", f"T={T}")


def test_gate_cumsum_varlen_short(kkt):
    inp = W.generate("T256_H8_bf16_f32", lengths=[1, 2, 3, 0, 64, 65, 0, 130, 5] + [1, 3] * 40, H=3, seed=2100)
    check(kkt, inp, "bf16", "varlen short")


def test_gate_cumsum_strong_decay_takes_the_clamp(kkt):
    """Decays of up to -3 per token: within-chunk gate differences reach
    about -96, beyond the clamp."""
    inp = W.generate("T256_H8_bf16_f32", T=200, H=2, seed=2200)
    rng = np.random.default_rng(2201)
    inp.g_raw = (-rng.uniform(0.0, 3.0, inp.g_raw.shape)).astype(np.float32)
    check(kkt, inp, "f32", "strong decay")


@pytest.mark.parametrize("in_dtype,out_dtype", [("f16", "f16"), ("f32", "bf16")])
def test_gate_cumsum_dtypes(kkt, in_dtype, out_dtype):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=150, H=3, in_dtype=in_dtype, seed=2300)
    check(kkt, inp, out_dtype, f"{in_dtype}->{out_dtype}")


@pytest.mark.parametrize("K,in_dtype,chunk", [(96, "bf16", 64), (160, "f32", 64), (32, "f16", 128), (192, "bf16", 128),
                                              (44, "f32", 64), (104, "bf16", 128)])
def test_gate_cumsum_head_dims(kkt, K, in_dtype, chunk):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=300, H=3, K=K, in_dtype=in_dtype, seed=2310 + K)
    check(kkt, inp, "f32", f"K={K} {in_dtype}", chunk=chunk)


def test_gate_cumsum_in_place_and_without_gate_output(kkt):
    """g_out == g_decay sums in place; leaving g_out NULL changes no row."""
    inp = W.generate("T256_H8_bf16_f32", B=2, T=300, H=5, seed=2400)
    say("[case] gate_cumsum in place / no gate output: B=2 T=300 H=5")
    ref_X, ref_g = run(kkt, inp, "f32")
    X_in, g_in = run(kkt, inp, "f32", in_place=True)
    X_none, _ = run(kkt, inp, "f32", with_gate_out=False)
    assert np.array_equal(g_in.view(np.uint32), ref_g.view(np.uint32))
    assert np.array_equal(X_in.view(np.uint32), ref_X.view(np.uint32))
    assert np.array_equal(X_none.view(np.uint32), ref_X.view(np.uint32))


def _run_g_out_at(kkt, inp: W.Inputs, offset: int):
    """The gate-sum op with g_out a view ``offset`` words into a larger
    buffer (offset 1: not 16-byte aligned)."""
    k, _g, b, cu = to_device(inp)
    a = torch.from_numpy(inp.g_raw).to(k.device)
    B, T, H, _ = k.shape
    out = torch.full((B, T, H, 64), float("nan"), dtype=torch.float32, device=k.device)
    buf = torch.full((B * T * H + 4,), float("nan"), dtype=torch.float32, device=k.device)
    g_out = buf[offset:offset + B * T * H].view(B, T, H)
    kkt.kkt_solve_gate_cumsum(k, a, b, cu, output_dtype=torch.float32, out=out, g_out=g_out)
    torch.cuda.synchronize()
    return from_device(out, "f32"), g_out.cpu().numpy()


@pytest.mark.parametrize("B,T,H", [(1, 65536 + 37, 4), (3, 22000, 8)])
def test_gate_cumsum_gathered_gate_stores(kkt, B, T, H):
    """Grids of more than 1024 four-wave workgroups, fixed-length rows, H a
    multiple of 4: each workgroup writes its four heads' summed gates
    together.  Against the oracle (a partial last chunk included), in place
    too, and bit-equal to the per-wave stores taken when g_out is not
    16-byte aligned."""
    inp = W.generate("T256_H8_bf16_f32", B=B, T=T, H=H, K=64, seed=2450 + H)
    assert B * -(-T // 64) * H > 4 * 1024
    check(kkt, inp, "f32", f"gathered B={B} T={T} H={H}")
    say(f"[case] gathered gate stores, in place and unaligned: B={B} T={T} H={H}")
    X_al, g_al = run(kkt, inp, "f32")
    X_in, g_in = run(kkt, inp, "f32", in_place=True)
    X_un, g_un = _run_g_out_at(kkt, inp, 1)
    for X, g in ((X_in, g_in), (X_un, g_un)):
        assert np.array_equal(X.view(np.uint32), X_al.view(np.uint32))
        assert np.array_equal(g.view(np.uint32), g_al.view(np.uint32))


@pytest.mark.parametrize("chunk", [64, 128])
def test_gate_cumsum_rising_and_wandering_decays(kkt, chunk):
    """Per-token log-decays of both signs (the summed gate rises and falls)
    and signed beta with zeros."""
    inp = W.generate("T256_H8_bf16_f32", B=2, T=700, H=4, seed=2460 + chunk)
    rng = np.random.default_rng(2461 + chunk)
    inp.g_raw = rng.uniform(-0.3, 0.3 if chunk == 64 else 0.2, inp.g_raw.shape).astype(np.float32)
    b = rng.uniform(-1.5, 1.5, inp.beta.shape)
    b[rng.random(b.shape) < 0.1] = 0.0
    inp.beta = b.astype(np.float32)
    check(kkt, inp, "f32", f"signed decays chunk={chunk}", chunk=chunk)


# ---------------------------------------------------------------- 128-token chunks
@pytest.mark.parametrize("name", GATED)
def test_gate_cumsum128_full_parity(kkt, name):
    inp = W.generate(name)
    check(kkt, inp, inp.workload.out_dtype, name, chunk=128)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 128, 129, 300])
def test_gate_cumsum128_lengths(kkt, T):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=T, H=3, seed=2500 + T, beta=bool(T % 2))
    check(kkt, inp, "f32", f"T={T}", chunk=128)


def test_gate_cumsum128_varlen_short(kkt):
    inp = W.generate("T256_H8_bf16_f32", lengths=[1, 2, 3, 0, 64, 65, 0, 130, 5, 128, 129, 300] + [1, 3] * 40,
                     H=3, seed=2600)
    check(kkt, inp, "bf16", "varlen short", chunk=128)


def test_gate_cumsum128_strong_decay_takes_the_clamp(kkt):
    inp = W.generate("T256_H8_bf16_f32", T=300, H=2, seed=2700)
    rng = np.random.default_rng(2701)
    inp.g_raw = (-rng.uniform(0.0, 3.0, inp.g_raw.shape)).astype(np.float32)
    check(kkt, inp, "f32", "strong decay", chunk=128)


@pytest.mark.parametrize("in_dtype,out_dtype,K", [("f16", "f16", 128), ("f32", "bf16", 128), ("bf16", "f32", 256),
                                                  ("f32", "f32", 64)])
def test_gate_cumsum128_dtypes_and_key_paths(kkt, in_dtype, out_dtype, K):
    """Keys shared through LDS (16-bit K <= 128, fp32 K = 64) and read by
    every wave (fp32 K = 128, 16-bit K = 256)."""
    inp = W.generate("T256_H8_bf16_f32", B=2, T=300, H=3, K=K, in_dtype=in_dtype, seed=2800 + K)
    check(kkt, inp, out_dtype, f"{in_dtype}->{out_dtype} K={K}", chunk=128)


def test_gate_cumsum128_in_place_and_without_gate_output(kkt):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=300, H=5, seed=2900)
    say("[case] gate_cumsum chunk=128 in place / no gate output: B=2 T=300 H=5")
    ref_X, ref_g = run(kkt, inp, "f32", chunk=128)
    X_in, g_in = run(kkt, inp, "f32", in_place=True, chunk=128)
    X_none, _ = run(kkt, inp, "f32", with_gate_out=False, chunk=128)
    assert np.array_equal(g_in.view(np.uint32), ref_g.view(np.uint32))
    assert np.array_equal(X_in.view(np.uint32), ref_X.view(np.uint32))
    assert np.array_equal(X_none.view(np.uint32), ref_X.view(np.uint32))
