"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle,
element by element on the same seeded inputs.

Every test needs a gfx950 GPU and the built library; none falls back to
anything.  Each case prints what it runs (and flushes) before touching the
GPU, so a log names the case if a run ends early.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from chunked_gated_delta_token_amd import workloads as W
from tests import _edge
from tests._compare import compare, fused_bound
from tests._gpu_util import TORCH_DT, from_device, load_kkt, say, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kkt():
    return load_kkt()


def run_gpu(kkt, inp: W.Inputs, out_dtype: str, stream=None, tensors=None) -> np.ndarray:
    k, g, b, cu = tensors if tensors is not None else to_device(inp)
    B, T, H, _ = k.shape
    out = torch.full((B, T, H, 64), float("nan"), dtype=TORCH_DT[out_dtype], device=k.device)
    kkt.kkt_solve(k, g, b, cu, output_dtype=TORCH_DT[out_dtype], out=out, stream=stream)
    torch.cuda.synchronize()
    return from_device(out, out_dtype)


def reference(inp: W.Inputs) -> np.ndarray:
    return oracle.kkt_solve_ref(inp.k64(), inp.g, inp.beta, inp.cu_seqlens)


def check_bits(kkt, inp: W.Inputs, out_dtype: str, label: str) -> np.ndarray:
    """check(), returning the GPU output."""
    w = inp.workload
    say(f"[case] {label}: B={w.B} T={w.T} H={w.H} K={w.K} in={w.in_dtype} out={out_dtype}")
    got = run_gpu(kkt, inp, out_dtype)
    ref = reference(inp)
    say("[ok] " + json.dumps(compare(got, ref, out_dtype, inp.cu_seqlens, label, fused_bound(inp, ref))))
    return got


def check(kkt, inp: W.Inputs, out_dtype: str, label: str) -> dict:
    w = inp.workload
    say(f"[case] {label}: B={w.B} T={w.T} H={w.H} K={w.K} in={w.in_dtype} out={out_dtype} "
        f"g={inp.g is not None} beta={inp.beta is not None} "
        f"seqs={0 if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1}")
    got = run_gpu(kkt, inp, out_dtype)
    ref = reference(inp)
    stats = compare(got, ref, out_dtype, inp.cu_seqlens, label, fused_bound(inp, ref))
    say("[ok] " + json.dumps(stats))
    return stats


# ---------------------------------------------------------------- full workloads
@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_parity(kkt, name):
    """Each workload at its full size, every output element compared."""
    inp = W.generate(name)
    check(kkt, inp, inp.workload.out_dtype, name)


# ---------------------------------------------------------------- dtype matrix
@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_dtype_matrix(kkt, in_dtype, out_dtype):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=200, H=3, in_dtype=in_dtype, seed=101)
    check(kkt, inp, out_dtype, f"dtype {in_dtype}->{out_dtype}")


# ---------------------------------------------------------------- shapes
@pytest.mark.parametrize("T", [1, 2, 3, 15, 16, 17, 63, 64, 65, 127, 128, 2000])
def test_lengths(kkt, T):
    gate, beta = bool(T % 2), bool((T // 2) % 2)
    inp = W.generate("T256_H8_bf16_f32", B=2, T=T, H=3, seed=200 + T, gate=gate, beta=beta)
    check(kkt, inp, "f32", f"T={T}")


@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("beta", [False, True])
def test_gate_beta_variants(kkt, gate, beta):
    inp = W.generate("T256_H8_bf16_f32", T=300, H=5, seed=300, gate=gate, beta=beta)
    check(kkt, inp, "f32", f"gate={gate} beta={beta}")
    check(kkt, inp, "bf16", f"gate={gate} beta={beta} bf16 out")


def _head_dim_case(kkt, K, in_dtype):
    inp = W.generate("T256_H8_bf16_f32", T=130, H=2, K=K, in_dtype=in_dtype, seed=400 + K)
    two = check_bits(kkt, inp, "f32", f"K={K} {in_dtype}")
    with kkt.option(kkt.KKT_OPTION_SPLIT_MAX_TILES, 0):
        one = run_gpu(kkt, inp, "f32")
    assert np.array_equal(one.view(np.uint32), two.view(np.uint32))


@pytest.mark.parametrize("K", [32, 64, 96, 160, 192, 224, 256])
@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "f32"])
def test_other_head_dims(kkt, K, in_dtype):
    """Every multiple of 32 up to 256 (K = 128 is every workload's): the
    kernels are built for 64, 128 and 256 and read the key pieces beyond a
    smaller K as zeros.  The grid (6 tiles) takes the two-wave tiles; the
    one-wave form is forced on the same inputs and must give the same bits."""
    _head_dim_case(kkt, K, in_dtype)


@pytest.mark.parametrize("K,in_dtype", [(4, "f32"), (36, "f32"), (68, "f32"), (100, "f32"), (132, "f32"),
                                        (252, "f32"), (8, "bf16"), (40, "bf16"), (72, "bf16"), (136, "bf16"),
                                        (248, "bf16"), (24, "f16"), (200, "f16")])
def test_head_dims_ending_inside_a_k_step(kkt, K, in_dtype):
    """K whose key rows end inside a 64-byte k-step (fp32: multiples of 4,
    bf16 / f16: multiples of 8): the lane groups whose 16-byte piece lies
    beyond K read zeros, the others their keys.  Both launch forms, same bits."""
    _head_dim_case(kkt, K, in_dtype)


@pytest.mark.parametrize("K", [96, 160, 40, 248])
def test_other_head_dims_one_wave_grid(kkt, K):
    """A K below its kernel's on a grid of one-wave tiles with bf16 output and
    packed sequences (the last key row of the last head ends the tensor, so
    the key resource must end at K, not at the kernel's K)."""
    inp = W.generate("T256_H8_bf16_f32", lengths=[900, 1, 64, 700, 63], H=3, K=K, seed=410 + K)
    check(kkt, inp, "bf16", f"packed K={K}")


def test_large_gate_spread(kkt):
    """Within-chunk gate differences beyond +-50 take the clamp."""
    inp = W.generate("T256_H8_bf16_f32", T=128, H=2, seed=450)
    rng = np.random.default_rng(451)
    inc = -rng.uniform(0.0, 3.0, inp.g.shape)
    g = np.empty_like(inc)
    for t0 in range(0, 128, 64):
        g[:, t0:t0 + 64] = np.cumsum(inc[:, t0:t0 + 64], axis=1)
    inp.g = g.astype(np.float32)
    check(kkt, inp, "f32", "gate spread ~ -96")


@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
@pytest.mark.parametrize("T,H", [(300, 3), (2400, 8)])
@pytest.mark.parametrize("kind", _edge.KINDS)
def test_edge_inputs(kkt, kind, T, H, out_dtype):
    """Signed and zero beta, rising or wandering gates, zero key rows and a
    zero chunk, on a two-wave grid (15 tiles) and a one-wave grid (304).  fp32 and f16
    output: the one-bf16-ulp rule is the one stated for decaying gates; with
    gates that rise, an element that nearly cancels in a chunk with |X| ~ 13
    measured 1.3e-7 off (fp32 arithmetic, fast exp), past that rule's
    2^-23 floor, and f16 output carries the fp32 error bound."""
    inp = _edge.edge_inputs(kind, T, H, seed=490 + T % 7)
    check(kkt, inp, out_dtype, f"{kind} T={T} H={H}")


@pytest.mark.parametrize("T,H", [(38481, 8), (40000, 7)])
def test_large_grid_tile_order(kkt, T, H):
    """Grids above 1024 workgroups take the chunk-grouped XCD order: these
    sizes leave a remainder of workgroups outside whole rounds, and with H=7
    the workgroups straddle chunks."""
    inp = W.generate("T256_H8_bf16_f32", T=T, H=H, seed=460 + H)
    check(kkt, inp, "bf16", f"large grid T={T} H={H}")


def test_many_heads(kkt):
    """H = 96 (not a power of two): 47 chunks x 24 workgroups per chunk, a grid
    above 1024 workgroups in the chunk-grouped order, with runs of 16
    workgroups and a remainder; row stride 24 KB."""
    inp = W.generate("T256_H8_bf16_f32", T=3000, H=96, seed=470)
    check(kkt, inp, "bf16", "many heads H=96")


@pytest.mark.parametrize("B,T,H,K,in_dtype,out_dtype", [
    (1, 1100, 1024, 16, "bf16", "bf16"),
    (1, 70, 4099, 8, "f16", "f32"),
    (1, 4000, 12, 256, "f32", "f32"),
])
def test_launch_fields_at_their_limits(kkt, B, T, H, K, in_dtype, out_dtype):
    """The launch fields the kernels receive packed into their first
    arguments, near the ends of their ranges: H = 1024 (18 chunks of 256
    four-wave workgroups, runs of 256 in the chunk-grouped order, whole
    rounds and a remainder, a 12-row last chunk); H = 4099 (odd: workgroups
    straddle chunks and the last one holds two tiles; a large magic number
    for the division by H; 16-byte key rows); 1 KB fp32 key rows (K = 256),
    the widest key row, on 756 one-wave tiles."""
    inp = W.generate("T256_H8_bf16_f32", B=B, T=T, H=H, K=K, in_dtype=in_dtype, seed=475 + H)
    check(kkt, inp, out_dtype, f"launch fields B={B} T={T} H={H} K={K}")


# ---------------------------------------------------------------- varlen
def _lengths(seed, n, lo, hi, empty_every=0):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=n)
    if empty_every:
        lens[::empty_every] = 0
    return [int(x) for x in lens]


VARLEN_CASES = {
    "tiny_and_empty": [1, 2, 3, 0, 64, 65, 0, 130, 5],
    "single": [777],
    "all_empty_but_one": [0, 0, 40, 0],
    "many_short": [1, 3] * 70,  # 140 sequences
    # the chunk lookup: one scan up to 64 sequences, beyond that a search
    # that narrows 64-fold per level (two levels up to 4096 sequences, three
    # beyond); cases on both sides of each step, with empty sequences among
    # them
    "one_level_64": _lengths(510, 64, 1, 70),
    "two_levels_65": _lengths(511, 65, 0, 70, empty_every=5),
    "two_levels_3000": _lengths(512, 3000, 0, 40, empty_every=7),
    "two_levels_4096": _lengths(513, 4096, 1, 20),
    "three_levels_4097": _lengths(514, 4097, 0, 20, empty_every=11),
}


@pytest.mark.parametrize("case", list(VARLEN_CASES))
def test_varlen(kkt, case):
    lens = VARLEN_CASES[case]
    inp = W.generate("T256_H8_bf16_f32", lengths=lens, H=3, seed=500)
    check(kkt, inp, "f32", f"varlen {case}")
    # the pages' split cross-check: the packed call equals one fixed-length
    # call per sequence, bit for bit
    packed = run_gpu(kkt, inp, "f32")
    cu = inp.cu_seqlens
    picked = range(len(lens)) if len(lens) <= 200 else sorted(set(range(0, len(lens), 97)) | {len(lens) - 1})
    for s in picked:
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        sub = W.Inputs(W.Workload(**{**inp.workload.__dict__, "T": b - a, "n_seqs": 0}),
                       np.ascontiguousarray(inp.k_store[:, a:b]),
                       None if inp.g is None else np.ascontiguousarray(inp.g[:, a:b]),
                       None if inp.beta is None else np.ascontiguousarray(inp.beta[:, a:b]), None)
        single = run_gpu(kkt, sub, "f32")
        assert np.array_equal(single.view(np.uint32), packed[:, a:b].view(np.uint32)), f"sequence {s}"


def test_varlen_validate_option_rejects_bad_offsets(kkt):
    """With KKT_OPTION_VALIDATE_CU_SEQLENS set, cu_seqlens is copied to the
    host and malformed offsets are rejected before anything is launched;
    valid offsets pass and give the same bits as without the check."""
    inp = W.generate("T256_H8_bf16_f32", lengths=[10, 20], H=2, seed=501)
    k, g, b, cu = to_device(inp)
    bad = torch.tensor([0, 25, 20], dtype=torch.int32, device=k.device)  # decreasing, ends != T
    plain = kkt.kkt_solve(k, g, b, cu, output_dtype=torch.float32)
    with kkt.option(kkt.KKT_OPTION_VALIDATE_CU_SEQLENS, 1):
        with pytest.raises(kkt.KKTError) as e:
            kkt.kkt_solve(k, g, b, bad)
        assert e.value.status == kkt.KKT_ERR_INVALID_ARGUMENT
        checked = kkt.kkt_solve(k, g, b, cu, output_dtype=torch.float32)
    assert kkt.get_option(kkt.KKT_OPTION_VALIDATE_CU_SEQLENS) == 0
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int32), checked.view(torch.int32))


def test_varlen_offsets_are_clamped(kkt):
    """Offsets beyond T are clamped in the kernel: rows inside [0, T) that a
    sequence covers are still correct and nothing outside the tensors is
    touched (the output's guard rows stay NaN)."""
    inp = W.generate("T256_H8_bf16_f32", lengths=[50, 30], H=2, seed=502)
    k, g, b, _ = to_device(inp)
    cu = torch.tensor([0, 50, 1000], dtype=torch.int32, device=k.device)  # last end beyond T=80
    guard = torch.full((1, 100, 2, 64), float("nan"), device=k.device)
    out = guard[:, :80]
    kkt.kkt_solve(k, g, b, cu, output_dtype=torch.float32, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(guard[:, 80:]).all()
    ref = reference(inp)
    compare(out.cpu().numpy(), ref, "f32", inp.cu_seqlens, "clamped offsets")


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("offsets", [
    [5, 3, 200, -7, 90, 80],     # decreasing, negative, beyond T
    [-10, 40, 20, 60],
    [30, 80],                    # not starting at 0: rows 0..29 belong to no sequence
    [79, 1, 0],
])
def test_varlen_malformed_offsets_stay_in_bounds(kkt, offsets, chunk):
    """Malformed offsets give unspecified rows but never a write outside the
    output: guard rows on both sides stay NaN, written rows are finite."""
    inp = W.generate("T256_H8_bf16_f32", T=80, H=2, seed=503)
    k, g, b, _ = to_device(inp)
    say(f"[case] malformed offsets {offsets} chunk={chunk}")
    cu = torch.tensor(offsets, dtype=torch.int32, device=k.device)
    guard = torch.full((1, 120, 2, chunk), float("nan"), device=k.device)
    out = guard[:, 20:100]
    kkt.kkt_solve(k, g, b, cu, chunk_size=chunk, output_dtype=torch.float32, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(guard[:, :20]).all() and torch.isnan(guard[:, 100:]).all()
    rows = out.cpu()
    written = ~torch.isnan(rows).all(dim=-1)
    assert torch.isfinite(rows[written]).all()
    if offsets == [30, 80]:
        assert not written[:, :30].any() and written[:, 30:].all()


# ---------------------------------------------------------------- bit-exact pins
def test_orthogonal_keys_give_identity(kkt):
    T, H, K = 192, 2, 64
    inp = W.generate("T256_H8_bf16_f32", T=T, H=H, K=K, seed=600)
    k = np.zeros((1, T, H, K))
    k[0, np.arange(T), :, np.arange(T) % 64] = 1.0
    inp.k_store = W.f64_to_bf16_bits(k)
    got = run_gpu(kkt, inp, "f32")
    eye = np.tile(np.eye(64, dtype=np.float32), (T // 64, 1))
    for h in range(H):
        assert np.array_equal(got[0, :, h].view(np.uint32), eye.view(np.uint32))


def test_beta_zero_gives_identity(kkt):
    inp = W.generate("T256_H8_bf16_f32", T=150, H=3, seed=601)
    inp.beta = np.zeros_like(inp.beta)
    got = run_gpu(kkt, inp, "bf16")
    local = np.arange(150) % 64
    exp = np.zeros((150, 64), dtype=np.uint16)
    exp[np.arange(150), local] = 0x3F80
    for h in range(3):
        assert np.array_equal(got[0, :, h], exp)


def test_single_token(kkt):
    inp = W.generate("T256_H8_bf16_f32", B=3, T=1, H=5, seed=602)
    got = run_gpu(kkt, inp, "f32")
    exp = np.zeros(64, dtype=np.float32)
    exp[0] = 1.0
    assert np.array_equal(got.reshape(-1, 64).view(np.uint32), np.tile(exp, (15, 1)).view(np.uint32))


def test_neutral_gate_beta_equal_null(kkt):
    inp = W.generate("T256_H8_bf16_f32", T=256, H=4, seed=603, gate=False, beta=False)
    a = run_gpu(kkt, inp, "f32")
    inp.g = np.zeros((1, 256, 4), dtype=np.float32)
    inp.beta = np.ones((1, 256, 4), dtype=np.float32)
    b = run_gpu(kkt, inp, "f32")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_head_and_batch_permutation(kkt):
    inp = W.generate("T256_H8_bf16_f32", B=2, T=200, H=4, seed=604)
    base = run_gpu(kkt, inp, "f32")
    p = np.array([3, 1, 0, 2])
    perm = W.Inputs(inp.workload, np.ascontiguousarray(inp.k_store[::-1][:, :, p]),
                    np.ascontiguousarray(inp.g[::-1][:, :, p]), np.ascontiguousarray(inp.beta[::-1][:, :, p]), None)
    got = run_gpu(kkt, perm, "f32")
    assert np.array_equal(got.view(np.uint32), base[::-1][:, :, p].view(np.uint32))


def test_prefix_partial_chunk_bitexact(kkt):
    """T=2000 against a T=2048 run sharing the first 2000 tokens: every row of
    the shorter run is bit-identical (a partial chunk is the leading block)."""
    full = W.generate("T256_H8_bf16_f32", T=2048, H=8, seed=605)
    part = W.Inputs(W.Workload(**{**full.workload.__dict__, "T": 2000}),
                    np.ascontiguousarray(full.k_store[:, :2000]), np.ascontiguousarray(full.g[:, :2000]),
                    np.ascontiguousarray(full.beta[:, :2000]), None)
    a = run_gpu(kkt, full, "f32")
    b = run_gpu(kkt, part, "f32")
    # columns >= 16 of the partial chunk are zero in the short run only
    assert np.array_equal(b[:, :1984].view(np.uint32), a[:, :1984].view(np.uint32))
    assert np.array_equal(b[:, 1984:, :, :16].view(np.uint32), a[:, 1984:2000, :, :16].view(np.uint32))
    assert np.all(b[:, 1984:, :, 16:].view(np.uint32) == 0)


def test_repeatable_and_stream(kkt):
    inp = W.generate("T8192_H8_bf16_f32")
    t = to_device(inp)
    a = run_gpu(kkt, inp, "f32", tensors=t)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_gpu(kkt, inp, "f32", stream=s, tensors=t)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_side_stream_noncontiguous_inputs(kkt):
    """A call on a stream other than the current one, with inputs that are
    strided views (so the binding copies them) produced on the current
    stream just before the call: the launch stream waits for the producer,
    the copies and the output are made on it, and the caller's tensors are
    recorded on it.  Every entry point gives the bits of the same call made
    on the current stream with contiguous inputs; the inputs are freed right
    after the call, before the side stream is synchronised."""
    inp = W.generate("T256_H8_bf16_f32", B=2, T=1500, H=6, seed=611)
    say("[case] side stream, transposed-view inputs: B=2 T=1500 H=6 K=128 bf16")
    k, g, b, _ = to_device(inp)
    ref = kkt.kkt_solve(k, g, b, output_dtype=torch.float32)
    ref_gs = kkt.kkt_solve_gate_cumsum(k, g, b, output_dtype=torch.float32, return_gate=True)
    ref_A = kkt.kkt_scaled_dot(k, g, b)
    ref_X = kkt.kkt_solve_tril(ref_A, output_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for rep in range(3):
        # produced on the current stream: [B,H,T,K] buffers viewed as [B,T,H,K]
        kt = torch.empty((k.shape[0], k.shape[2], k.shape[1], k.shape[3]), dtype=k.dtype, device=k.device)
        kt.copy_(k.permute(0, 2, 1, 3))
        gt = torch.empty((g.shape[0], g.shape[2], g.shape[1]), dtype=g.dtype, device=g.device)
        gt.copy_(g.permute(0, 2, 1))
        bt = torch.empty_like(gt)
        bt.copy_(b.permute(0, 2, 1))
        At = torch.empty((ref_A.shape[0], ref_A.shape[2], ref_A.shape[1], 64), dtype=torch.float32, device=k.device)
        At.copy_(ref_A.permute(0, 2, 1, 3))
        kv, gv, bv, Av = kt.permute(0, 2, 1, 3), gt.permute(0, 2, 1), bt.permute(0, 2, 1), At.permute(0, 2, 1, 3)
        assert not kv.is_contiguous()
        x = kkt.kkt_solve(kv, gv, bv, output_dtype=torch.float32, stream=s)
        xg, gg = kkt.kkt_solve_gate_cumsum(kv, gv, bv, output_dtype=torch.float32, return_gate=True, stream=s)
        A = kkt.kkt_scaled_dot(kv, gv, bv, stream=s)
        X = kkt.kkt_solve_tril(Av, output_dtype=torch.bfloat16, stream=s)
        del kt, gt, bt, At, kv, gv, bv, Av
        # new work on the current stream may now reuse freed memory
        junk = [torch.full((1 << 20,), float("nan"), device=k.device) for _ in range(8)]
        s.synchronize()
        del junk
        for got, want in ((x, ref), (xg, ref_gs[0]), (gg, ref_gs[1]), (A, ref_A)):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), f"rep {rep}"
        assert torch.equal(X.view(torch.int16), ref_X.view(torch.int16)), f"rep {rep}"


def test_concurrent_host_threads(kkt):
    """Four host threads, each with its own stream and its own entry point
    (64- and 128-token chunks, the gate-sum entry and the two-step chain),
    launch 25 calls each at the same time; every result equals the same
    call made alone, bit for bit."""
    import threading
    inp = W.generate("T256_H8_bf16_f32", B=2, T=1000, H=6, seed=610)
    say("[case] concurrent host threads: 4 threads x 25 calls")
    k, g, b, cu = to_device(inp)
    B, T, H, _ = k.shape
    dev = k.device

    def jobs():
        out = {
            "fused64": torch.empty((B, T, H, 64), dtype=torch.float32, device=dev),
            "fused128": torch.empty((B, T, H, 128), dtype=torch.bfloat16, device=dev),
            "gate_cumsum": torch.empty((B, T, H, 64), dtype=torch.float16, device=dev),
            "chain_A": torch.empty((B, T, H, 64), dtype=torch.float32, device=dev),
            "chain": torch.empty((B, T, H, 64), dtype=torch.float32, device=dev),
        }
        decay = g.clone()
        calls = {
            "fused64": lambda s: kkt.kkt_solve(k, g, b, output_dtype=torch.float32, out=out["fused64"], stream=s),
            "fused128": lambda s: kkt.kkt_solve(k, g, b, chunk_size=128, output_dtype=torch.bfloat16,
                                                out=out["fused128"], stream=s),
            "gate_cumsum": lambda s: kkt.kkt_solve_gate_cumsum(k, decay, b, output_dtype=torch.float16,
                                                               out=out["gate_cumsum"], stream=s),
            "chain": lambda s: (kkt.kkt_scaled_dot(k, g, b, out=out["chain_A"], stream=s),
                                kkt.kkt_solve_tril(out["chain_A"], output_dtype=torch.float32, out=out["chain"],
                                                   stream=s)),
        }
        return out, calls

    alone, alone_calls = jobs()
    s0 = torch.cuda.Stream()
    for fn in alone_calls.values():
        fn(s0)
    torch.cuda.synchronize()
    together, calls = jobs()
    errors = []

    def worker(name):
        try:
            s = torch.cuda.Stream()
            for _ in range(25):
                calls[name](s)
            s.synchronize()
        except Exception as e:  # noqa: BLE001  (reported below)
            errors.append((name, repr(e)))

    threads = [threading.Thread(target=worker, args=(n,)) for n in calls]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for name in ("fused64", "fused128", "gate_cumsum", "chain"):
        a, b2 = alone[name], together[name]
        bits = torch.int32 if a.dtype == torch.float32 else torch.int16
        assert torch.equal(a.view(bits), b2.view(bits)), name


def test_graph_capture_replays(kkt):
    """kkt_solve captured in a HIP graph (the library launches one kernel and
    records no memset): every replay, with eager work and synchronisations in
    between, equals the eager result bit for bit, also after the inputs
    change in place."""
    inp = W.generate("T2000_H8_bf16_bf16")
    say("[case] graph capture: T2000_H8 bf16 -> bf16, 4 replays")
    k, g, b, cu = to_device(inp)
    B, T, H, _ = k.shape
    out = torch.empty((B, T, H, 64), dtype=torch.bfloat16, device=k.device)
    eager = torch.empty_like(out)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        kkt.kkt_solve(k, g, b, output_dtype=torch.bfloat16, out=eager, stream=s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        kkt.kkt_solve(k, g, b, output_dtype=torch.bfloat16, out=out, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
        if rep == 1:  # new values in the captured input buffers
            k.mul_(-1.0)
            with torch.cuda.stream(s):
                kkt.kkt_solve(k, g, b, output_dtype=torch.bfloat16, out=eager, stream=s)
            torch.cuda.synchronize()


# ---------------------------------------------------------------- golden file on the GPU
def test_hand_worked_golden_on_gpu(kkt):
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_chunks.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        kk = np.array(c["k"], dtype=np.float64)
        T, Kc = kk.shape
        k = np.zeros((1, T, 1, 64))
        k[0, :, 0, :Kc] = kk           # zero padding keeps every dot product
        wl = W.Workload("golden", 1, T, 1, 64, "f32", "f32", c["g"] is not None, c["beta"] is not None, 0)
        inp = W.Inputs(wl, k.astype(np.float32),
                       None if c["g"] is None else np.array(c["g"], dtype=np.float32).reshape(1, T, 1),
                       None if c["beta"] is None else np.array(c["beta"], dtype=np.float32).reshape(1, T, 1),
                       None if c["cu_seqlens"] is None else np.array(c["cu_seqlens"], dtype=np.int32))
        got = run_gpu(kkt, inp, "f32")
        for t, row in enumerate(c["expected_rows"]):
            exp = np.zeros(64)
            exp[:len(row)] = row
            # fp32 exp of an argument x carries a relative error of about
            # |x| log2(e) 2^-24 (the clamp case has x = 50: ~4.3e-6), so the
            # fp32 kernel is held to the 1e-5 relative bar of the criteria
            tol = 1e-5 * np.maximum(np.abs(exp), 1.0)
            assert np.all(np.abs(got[0, t, 0] - exp) <= tol), (c["name"], t, got[0, t, 0, :4])


# ---------------------------------------------------------------- error paths
def test_error_paths(kkt):
    inp = W.generate("T256_H8_bf16_f32", T=64, H=1, seed=700)
    k, g, b, _ = to_device(inp)
    with pytest.raises(ValueError):
        kkt.kkt_solve(k, g, b, chunk_size=256)
    out = torch.empty((1, 64, 1, 64), device=k.device)
    for kwargs, status in (
        (dict(chunk_size=32), kkt.KKT_ERR_UNSUPPORTED),
        (dict(K=100), kkt.KKT_ERR_UNSUPPORTED),
        (dict(in_dtype=7), kkt.KKT_ERR_INVALID_ARGUMENT),
        (dict(B=0), kkt.KKT_ERR_INVALID_ARGUMENT),
    ):
        args = dict(chunk_size=64, K=128, in_dtype=1, B=1)
        args.update(kwargs)
        st = kkt.kkt_solve_raw(k.data_ptr(), g.data_ptr(), b.data_ptr(), None, 0, args["B"], 64, 1, args["K"],
                               args["chunk_size"], args["in_dtype"], 0, out.data_ptr(), None)
        assert st == status, (kwargs, st, kkt.last_error())
        assert kkt.last_error()


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_16bit_output_is_rne_of_fp32_output(kkt, out_dtype):
    """The 16-bit outputs are the kernel's own fp32 results rounded to nearest
    even, bit for bit (same inputs, same arithmetic up to the store)."""
    inp = W.generate("T256_H8_bf16_f32", B=2, T=300, H=5, seed=650)
    f32 = run_gpu(kkt, inp, "f32")
    got = run_gpu(kkt, inp, out_dtype)
    if out_dtype == "bf16":
        exp = oracle.round_to_bf16_bits(f32.astype(np.float64))
    else:
        exp = f32.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, exp), int(np.sum(got != exp))
