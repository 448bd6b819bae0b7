"""Benchmark of the fused chunk-local KKT + triangular solve on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]

One step = one call of the fused op (the whole hot path: tile map, K load,
Gram, gate/beta epilogue, diagonal solve, block merge, store) over one batch
of synthetic inputs of the bench workload, (B,T,H,K) = (1,8192,8,128) with
bf16 keys and fp32 output.  Inputs are resident in HBM before the timed
region starts.  Successive steps rotate over R copies of the input and output
buffers whose total size exceeds twice the 256 MB Infinity Cache, so every
step reads its keys from HBM.

Timed region: K steps captured in one HIP graph (launch overhead of the
Python/ctypes call path is not the op's), bracketed by a device
synchronisation and HIP events on the launch stream.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused KKT+solve ms/iter & achieved HBM GB/s at (1,8192,8,128) bf16, 1 GPU"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak
PAGES_FUSED_MS = 0.3593         # Ascend 910B fused op at (1,8192,8,128), PR #135 perf table (context only)
MALL_BYTES = 256 << 20
KERNEL_SRC = os.path.join(ROOT, "chunked_gated_delta_token_amd", "csrc", "kkt_solve.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_kkt_solve_T8192_H8_bf16_f32.txt")

ESIZE = {"f32": 4, "bf16": 2, "f16": 2}


def algorithmic_bytes(w, n_tokens: int) -> int:
    """Minimum bytes one call must move: k once, g and beta once (when given),
    the output once.  (cu_seqlens, a few bytes, is ignored.)"""
    H, K = w.H, w.K
    per_token = H * K * ESIZE[w.in_dtype] + H * 64 * ESIZE[w.out_dtype]
    per_token += H * 4 * (int(w.gate) + int(w.beta))
    return per_token * n_tokens


def source_digest() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(digest: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; None otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, nbytes: int, budget_s: float):
    """The fp64 oracle (as it is) on the same workload, repeated until about
    budget_s seconds of CPU work; throughput in the metric's unit."""
    import oracle
    k64, g, b = inp.k64(), inp.g, inp.beta
    g64 = None if g is None else g.astype("float64")
    b64 = None if b is None else b.astype("float64")
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.kkt_solve_ref(k64, g64, b64, inp.cu_seqlens)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": nbytes * reps / el / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole workload, {reps} calls in {el:.1f} s (fp64, OpenMP over chunk-head tiles)"}


def copy_calibration(nbytes: int, steps: int):
    """Plain device-to-device copies of a known size, over buffers rotated
    past the Infinity Cache: under rocprofv3 --pmc they give the counter
    reading per byte actually read / written."""
    import torch
    n = nbytes // 4
    R = max(2, -(-2 * MALL_BYTES // (2 * nbytes)))
    src = [torch.ones(n, device="cuda") for _ in range(R)]
    dst = [torch.empty(n, device="cuda") for _ in range(R)]
    for i in range(steps):
        dst[i % R].copy_(src[i % R])
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "steps": steps, "buffer_sets": R}), flush=True)


def _counter_values(directory: str, counter: str, kernel_substr: str):
    """Per-dispatch values of one counter for kernels whose name contains
    kernel_substr, from a rocprofv3 --pmc CSV output directory."""
    import csv
    import glob
    vals = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter and kernel_substr in row.get("Kernel_Name", ""):
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} values for '{kernel_substr}' under {directory}")
    return vals


def summarize_traffic(dirs, copy_bytes: int):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the op, each scaled by
    the bytes-per-KiB ratio the same counter shows for a plain copy."""
    import statistics
    if copy_bytes <= 0:
        raise SystemExit("--copy-bytes is required")
    op_fetch = statistics.median(_counter_values(dirs[0], "FETCH_SIZE", "kkt_solve_kernel"))
    op_write = statistics.median(_counter_values(dirs[1], "WRITE_SIZE", "kkt_solve_kernel"))
    cp_fetch = statistics.median(_counter_values(dirs[2], "FETCH_SIZE", "copy"))
    cp_write = statistics.median(_counter_values(dirs[3], "WRITE_SIZE", "copy"))
    f_scale = copy_bytes / cp_fetch
    w_scale = copy_bytes / cp_write
    fetch_b, write_b = op_fetch * f_scale, op_write * w_scale
    lines = [
        "# HBM traffic of kkt_solve_kernel, bench workload T8192_H8_bf16_f32 (B=1,T=8192,H=8,K=128 bf16 -> fp32)",
        "# commands (run from the repository root, then summarized by the last one):",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <op_fetch> -- python bench.py --timing eager --steps 20 --warmup 2 --no-cpu-baseline",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <op_write> -- python bench.py --timing eager --steps 20 --warmup 2 --no-cpu-baseline",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <copy_fetch> -- python bench.py --copy-calibration {copy_bytes} --steps 20",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <copy_write> -- python bench.py --copy-calibration {copy_bytes} --steps 20",
        f"#   python bench.py --summarize-traffic <op_fetch> <op_write> <copy_fetch> <copy_write> --copy-bytes {copy_bytes}",
        f"kernel_source_sha256_16: {source_digest()}",
        f"op_fetch_size_kib_median: {op_fetch:.1f}",
        f"op_write_size_kib_median: {op_write:.1f}",
        f"copy_bytes: {copy_bytes}",
        f"copy_fetch_size_kib_median: {cp_fetch:.1f}",
        f"copy_write_size_kib_median: {cp_write:.1f}",
        f"fetch_bytes_per_kib: {f_scale:.2f}",
        f"write_bytes_per_kib: {w_scale:.2f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
    ]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--timing", choices=["graph", "eager"], default="graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail", action="store_true", help="also print per-launch event timings to stderr")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the op, run --steps plain device copies of BYTES bytes (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("OP_FETCH", "OP_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the HBM-traffic summary from four rocprofv3 --pmc output directories")
    ap.add_argument("--copy-bytes", type=int, default=0, help="size used by the copy-calibration runs")
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.copy_bytes)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the fused KKT + solve has no cross-GPU step, and this "
              "build runs on a single MI355X (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return

    from chunked_gated_delta_token_amd import kkt
    from chunked_gated_delta_token_amd import workloads as W

    name = args.workload or W.BENCH_WORKLOAD
    inp = W.generate(name)
    w = inp.workload
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = kkt.load_library()

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    kdt = {"f32": kkt.KKT_DTYPE_F32, "bf16": kkt.KKT_DTYPE_BF16, "f16": kkt.KKT_DTYPE_F16}
    if w.in_dtype == "f32":
        k0 = torch.from_numpy(inp.k_store).to(dev)
    else:
        k0 = torch.from_numpy(inp.k_store.view(np.int16)).to(dev).view(tdt[w.in_dtype])
    g0 = None if inp.g is None else torch.from_numpy(inp.g).to(dev)
    b0 = None if inp.beta is None else torch.from_numpy(inp.beta).to(dev)
    cu0 = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to(dev)
    n_tokens = w.B * w.T
    nbytes = algorithmic_bytes(w, n_tokens)
    R = max(2, -(-2 * MALL_BYTES // nbytes))
    sets = []
    for _ in range(R):
        sets.append(dict(k=k0.clone(), g=None if g0 is None else g0.clone(), b=None if b0 is None else b0.clone(),
                         cu=None if cu0 is None else cu0.clone(),
                         out=torch.empty((w.B, w.T, w.H, 64), dtype=tdt[w.out_dtype], device=dev)))
    del k0, g0, b0
    stream = torch.cuda.Stream(dev)
    num_seqs = 0 if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1

    def ptr(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    calls = [(ptr(s["k"]), ptr(s["g"]), ptr(s["b"]), ptr(s["cu"]), num_seqs, w.B, w.T, w.H, w.K, 64,
              kdt[w.in_dtype], kdt[w.out_dtype], ptr(s["out"]), ctypes.c_void_p(stream.cuda_stream)) for s in sets]

    def launch(i):
        st = lib.kkt_solve(*calls[i % R])
        if st != 0:
            raise RuntimeError(f"kkt_solve status {st}: {kkt.last_error()}")

    # correctness guard on the bench inputs (cheap structural check, no oracle)
    with torch.cuda.stream(stream):
        launch(0)
    torch.cuda.synchronize()
    o = sets[0]["out"].float()
    assert torch.isfinite(o).all().item(), "non-finite output"
    del o

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()

    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph = None
    if args.timing == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream, capture_error_mode="thread_local"):
            for i in range(K):
                launch(i)
        with torch.cuda.stream(stream):
            graph.replay()  # first replay uploads the graph; not timed
        torch.cuda.synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):  # a graph replays on the current stream
        ev0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(K):
                launch(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / K
    ms_per_step = wall * 1e3 / K

    detail = {}
    if args.detail:
        # per-launch event pairs (eager), for comparison with the profiler
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(64)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(64)]
        for i in range(64):
            starts[i].record(stream)
            launch(i)
            ends[i].record(stream)
        torch.cuda.synchronize()
        per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
        detail = {"per_launch_event_ms_median": per[len(per) // 2], "per_launch_event_ms_min": per[0],
                  "graph_event_ms": ev_ms, "wall_ms": ms_per_step}
        print(json.dumps(detail), file=sys.stderr, flush=True)

    achieved = nbytes / (ev_ms * 1e-3) / 1e9
    digest = source_digest()
    traffic = read_traffic(digest)
    n_tiles = w.H * (sum(-(-(int(inp.cu_seqlens[s + 1]) - int(inp.cu_seqlens[s])) // 64)
                         for s in range(num_seqs)) if num_seqs else w.B * (-(-w.T // 64)))
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(PAGES_FUSED_MS / ms_per_step, 3) if name == W.BENCH_WORKLOAD else None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "in_dtype": w.in_dtype,
                   "out_dtype": w.out_dtype, "gate": w.gate, "beta": w.beta, "tiles": n_tiles,
                   "algorithmic_bytes": nbytes, "buffer_sets": R, "timing": args.timing,
                   "chunks_per_s": round(n_tiles / (ms_per_step * 1e-3), 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "event_ms_per_launch": round(ev_ms, 6), "kernel_source_sha256_16": digest},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, nbytes, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
