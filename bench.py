"""Benchmark of the fused chunk-local KKT + triangular solve on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--op OP]

One step = one call of the fused op (the whole hot path: tile map, K load,
Gram, gate/beta epilogue, diagonal solve, block merge, store) over one batch
of synthetic inputs of the bench workload, (B,T,H,K) = (1,8192,8,128) with
bf16 keys and fp32 output.  Inputs are resident in HBM before the timed
region starts.  Successive steps rotate over R copies of the input and output
buffers whose total size exceeds twice the 256 MB Infinity Cache, so every
step reads its keys from HBM.

--op picks what one step is: the fused op (default), or one step of the
unfused two-step chain on its own (scaled_dot: k, g, beta -> A in fp32;
solve_tril: A -> (I+A)^{-1}), or the whole chain (both launches, A through
HBM), or the memory-traffic reference (floor: libkkt_floor.so's kernel,
which moves the fused op's bytes in its access pattern with no arithmetic;
sequences of whole 64-token chunks only).

Timed region: K steps captured in one HIP graph (launch overhead of the
Python/ctypes call path is not the op's), bracketed by a device
synchronisation and HIP events on the launch stream.  Prints one JSON line.

The default run (the fused op on the bench workload) also times the second
shape of the PR #135 table that the target names, (2,16384,32,128) bf16 keys
and bf16 output, the same way in the same process, and reports it under
"second_target" (the headline fields stay those of (1,8192,8,128)).
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
PAGES_TWO_OP_MS = 0.4318        # Ascend 910B two-op chain at (1,8192,8,128), same table (context only)
PAGES_FUSED_MS_SECOND = 4.9368  # Ascend 910B fused op at (2,16384,32,128), same table (context only)
MALL_BYTES = 256 << 20
KERNEL_SRC = os.path.join(ROOT, "chunked_gated_delta_token_amd", "csrc", "kkt_solve.hip")
# the kernel each op launches (chain: both of the unfused steps)
KERNELS = {"fused": "kkt_solve_kernel", "scaled_dot": "kkt_scaled_dot_kernel",
           "solve_tril": "kkt_solve_tril_kernel", "chain": "kkt_scaled_dot_kernel+kkt_solve_tril_kernel",
           "gate_cumsum": "kkt_solve_gate_cumsum_kernel", "fused128": "kkt_solve128_kernel",
           "gate_cumsum128": "kkt_solve128_kernel", "floor": "stream_floor_kernel"}
# names of the profile files (fused128 / gate_cumsum128: those ops with 128-token chunks)
ENTRY = {"fused": "kkt_solve", "scaled_dot": "kkt_scaled_dot", "solve_tril": "kkt_solve_tril",
         "gate_cumsum": "kkt_solve_gate_cumsum", "fused128": "kkt_solve128",
         "gate_cumsum128": "kkt_solve_gate_cumsum128", "floor": "stream_floor"}


SPLIT_MAX_TILES = 256          # the library's own bound for two-wave tiles (KKT_SPLIT_TILES >= 0 overrides it)


def kernel_name(key: str, workload: str) -> str:
    """The kernel an op key launches on a workload: the fused op at 64-token
    chunks (with or without the gate sum) and the solve of a given A take
    their two-wave-per-tile form on grids of up to SPLIT_MAX_TILES
    chunk-head tiles (the library's grid counts T/64 + num_seqs chunks for
    packed sequences), except the fused op with 16-bit keys and output,
    which the library keeps at one wave per tile unless KKT_SPLIT_TILES
    sets a bound."""
    from chunked_gated_delta_token_amd import workloads as W
    split_names = {"fused": "kkt_solve_split_kernel", "gate_cumsum": "kkt_solve_gate_cumsum_split_kernel",
                   "solve_tril": "kkt_solve_tril_split_kernel"}
    if key in split_names:
        w = W.WORKLOADS[workload]
        grid = w.H * ((w.T // 64 + w.n_seqs) if w.n_seqs else w.B * (-(-w.T // 64)))
        env = os.environ.get("KKT_SPLIT_TILES", "")
        bound = int(env) if env else -1
        if bound < 0:
            sixteen_bit = w.in_dtype != "f32" and w.out_dtype != "f32"
            bound = 0 if (key == "fused" and sixteen_bit) else SPLIT_MAX_TILES
        if grid <= bound:
            return split_names[key]
    return KERNELS[key]


def op_key(op: str, chunk: int) -> str:
    return op + "128" if (op in ("fused", "gate_cumsum") and chunk == 128) else op


def traffic_file(op: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{ENTRY[op]}_{workload}.txt")


ESIZE = {"f32": 4, "bf16": 2, "f16": 2}


def chunk_lengths(w, cu_seqlens):
    """Lengths L of every chunk of one head."""
    if cu_seqlens is None:
        full, tail = divmod(w.T, 64)
        return [64] * full * w.B + ([tail] * w.B if tail else [])
    out = []
    for s in range(len(cu_seqlens) - 1):
        n = int(cu_seqlens[s + 1]) - int(cu_seqlens[s])
        out += [64] * (n // 64) + ([n % 64] if n % 64 else [])
    return out


def algorithmic_bytes(w, n_tokens: int, op: str = "fused", cu_seqlens=None, chunk: int = 64) -> int:
    """Minimum bytes one step must move.  fused and chain: k once, g and beta
    once (when given), the output once (the chain's A round trip is its own
    overhead, not the step's work); with 128-token chunks the output rows are
    128 wide.  gate_cumsum: as fused, plus the summed
    gate written back.  scaled_dot: k, g, beta, and A in fp32.
    solve_tril: the strictly lower entries of A (L (L-1) / 2 fp32 values per
    chunk and head) and the output.  (cu_seqlens, a few bytes, is ignored.)"""
    H, K = w.H, w.K
    k_gb = H * K * ESIZE[w.in_dtype] + H * 4 * (int(w.gate) + int(w.beta))
    out = H * chunk * ESIZE[w.out_dtype]
    if op in ("fused", "chain", "floor"):
        return (k_gb + out) * n_tokens
    if op == "gate_cumsum":
        return (k_gb + out + H * 4) * n_tokens
    if op == "scaled_dot":
        return (k_gb + H * 64 * 4) * n_tokens
    lower = sum(L * (L - 1) // 2 for L in chunk_lengths(w, cu_seqlens)) * 4 * H
    return lower + out * n_tokens


FLOOR_LIB = os.path.join(ROOT, "chunked_gated_delta_token_amd", "libkkt_floor.so")


def load_floor():
    """kkt_floor_copy from the in-tree libkkt_floor.so (raises if it is not built)."""
    if not os.path.exists(FLOOR_LIB):
        raise SystemExit(f"{FLOOR_LIB} is missing: build it with `python -m chunked_gated_delta_token_amd.build`")
    lib = ctypes.CDLL(FLOOR_LIB)
    fn = lib.kkt_floor_copy
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    return fn


FLOOR_SRC = os.path.join(ROOT, "chunked_gated_delta_token_amd", "csrc", "stream_floor.hip")


def source_digest(op: str = "fused") -> str:
    """Digest of the source of the kernel an op runs (the memory-traffic
    reference has its own source file)."""
    with open(FLOOR_SRC if op == "floor" else KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(digest: str, path: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; None otherwise."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
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


def cpu_baseline(inp, nbytes: int, budget_s: float, op: str = "fused", chunk: int = 64):
    """The fp64 oracle (as it is) for the same step on the same workload,
    repeated until about budget_s seconds of CPU work; throughput in the
    metric's unit."""
    import oracle
    k64, g, b, cu = inp.k64(), inp.g, inp.beta, inp.cu_seqlens
    g64 = None if g is None else g.astype("float64")
    b64 = None if b is None else b.astype("float64")
    A = None
    if op == "solve_tril":
        A = oracle.scaled_dot_ref(k64, g64, b64, cu).astype("float32").astype("float64")
    reps, t0 = 0, time.perf_counter()
    while True:
        if op == "fused":
            oracle.kkt_solve_ref(k64, g64, b64, cu, chunk_size=chunk)
        elif op == "gate_cumsum":
            oracle.kkt_solve_gate_cumsum_ref(k64, inp.g_raw, b64, cu, chunk_size=chunk)
        elif op == "scaled_dot":
            oracle.scaled_dot_ref(k64, g64, b64, cu)
        elif op == "solve_tril":
            oracle.solve_tril_ref(A, cu)
        else:
            oracle.solve_tril_ref(oracle.scaled_dot_ref(k64, g64, b64, cu), cu)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    what = {"fused": "the fused op", "scaled_dot": "A alone", "solve_tril": "the solve of a given A",
            "chain": "A, then its solve", "gate_cumsum": "gate sum, then the fused op"}[op]
    threads = oracle.num_threads()
    out = {"value": nbytes * reps / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole workload ({what}), {reps} calls in {el:.1f} s (fp64, OpenMP over chunk-head tiles)",
           "cpu": cpu_model()}
    if op == "fused":
        # the same on one thread, over a shorter sample
        oracle.set_num_threads(1)
        try:
            reps1, t1 = 0, time.perf_counter()
            while True:
                oracle.kkt_solve_ref(k64, g64, b64, cu, chunk_size=chunk)
                reps1 += 1
                el1 = time.perf_counter() - t1
                if el1 >= budget_s / 3:
                    break
        finally:
            oracle.set_num_threads(threads)
        out["single_thread_value"] = nbytes * reps1 / el1 / 1e9
        out["single_thread_sample"] = f"{reps1} calls in {el1:.1f} s"
    return out


def cpu_model() -> str:
    """The host CPU's model name and logical CPU count (Linux)."""
    try:
        with open("/proc/cpuinfo") as f:
            names = [l.split(":", 1)[1].strip() for l in f if l.startswith("model name")]
        return f"{names[0]} ({len(names)} logical CPUs)" if names else "unknown"
    except OSError:
        return "unknown"


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


def summarize_traffic(dirs, copy_bytes: int, op: str, workload: str, chunk: int = 64):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the op's kernel, each
    scaled by the bytes-per-KiB ratio the same counter shows for a plain copy."""
    import statistics
    if copy_bytes <= 0:
        raise SystemExit("--copy-bytes is required")
    if op == "chain":
        raise SystemExit("traffic is summarized per kernel: use --op fused, gate_cumsum, scaled_dot or solve_tril")
    key = op_key(op, chunk)
    kname = kernel_name(key, workload)
    op_fetch = statistics.median(_counter_values(dirs[0], "FETCH_SIZE", kname))
    op_write = statistics.median(_counter_values(dirs[1], "WRITE_SIZE", kname))
    cp_fetch = statistics.median(_counter_values(dirs[2], "FETCH_SIZE", "copy"))
    cp_write = statistics.median(_counter_values(dirs[3], "WRITE_SIZE", "copy"))
    f_scale = copy_bytes / cp_fetch
    w_scale = copy_bytes / cp_write
    fetch_b, write_b = op_fetch * f_scale, op_write * w_scale
    sel = f"--op {op} --workload {workload}" + (f" --chunk {chunk}" if chunk != 64 else "")
    lines = [
        f"# HBM traffic of {kname}, workload {workload}",
        "# commands (from /tmp, repository at $R; each --pmc pass alone, the last command wrote this file):",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <op_fetch> -o p -- python -u $R/bench.py {sel} --timing eager --steps 20 --warmup 2 --no-cpu-baseline --no-second-target --no-floor",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <op_write> -o p -- python -u $R/bench.py {sel} --timing eager --steps 20 --warmup 2 --no-cpu-baseline --no-second-target --no-floor",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <copy_fetch> -o p -- python -u $R/bench.py --copy-calibration {copy_bytes} --steps 20",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <copy_write> -o p -- python -u $R/bench.py --copy-calibration {copy_bytes} --steps 20",
        f"#   python $R/bench.py --summarize-traffic <op_fetch> <op_write> <copy_fetch> <copy_write> --copy-bytes {copy_bytes} {sel}",
        f"kernel_source_sha256_16: {source_digest(op)}",
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
    path = traffic_file(key, workload)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F32")
N_SIMDS = 256 * 4               # MI355X: 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9                # MI355X peak engine clock


def mfma_file(op: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"mfma_{ENTRY[op]}_{workload}.txt")


def summarize_mfma(directory: str, op: str, workload: str, chunk: int = 64):
    """Matrix-core counters of the op's kernel from one rocprofv3 --pmc pass:
    MFMA busy cycles (summed over SIMDs) and MFMA operations (units of 512
    flop) per launch, medians over the launches."""
    import statistics
    key = op_key(op, chunk)
    kname = kernel_name(key, workload)
    med = {c: statistics.median(_counter_values(directory, c, kname)) for c in MFMA_COUNTERS}
    sel = f"--op {op} --workload {workload}" + (f" --chunk {chunk}" if chunk != 64 else "")
    lines = [
        f"# MFMA counters of {kname}, workload {workload} (medians per launch)",
        "# commands (from /tmp, repository at $R; the last one wrote this file):",
        f"#   rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv -d <dir> -o p -- python -u $R/bench.py "
        f"{sel} --timing eager --steps 10 --warmup 2 --no-cpu-baseline --no-second-target --no-floor",
        f"#   python $R/bench.py --summarize-mfma <dir> {sel}",
        "# busy cycles are summed over the SIMDs; one MFMA operation (MOPS) is 512 flop",
        f"kernel_source_sha256_16: {source_digest(op)}",
        f"mfma_busy_cycles_per_launch: {med['SQ_VALU_MFMA_BUSY_CYCLES']:.0f}",
        f"mfma_flop_bf16_per_launch: {512 * med['SQ_INSTS_VALU_MFMA_MOPS_BF16']:.0f}",
        f"mfma_flop_f16_per_launch: {512 * med['SQ_INSTS_VALU_MFMA_MOPS_F16']:.0f}",
        f"mfma_flop_f32_per_launch: {512 * med['SQ_INSTS_VALU_MFMA_MOPS_F32']:.0f}",
    ]
    path = mfma_file(key, workload)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_mfma(digest: str, path: str):
    """The counter summary's values, if taken on the current kernel source."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != digest:
        return None
    try:
        return {k: float(vals[k]) for k in ("mfma_busy_cycles_per_launch", "mfma_flop_bf16_per_launch",
                                            "mfma_flop_f16_per_launch", "mfma_flop_f32_per_launch")}
    except (KeyError, ValueError):
        return None


def summarize_trace(directory: str, op: str, workload: str, run_log: str = None, plain_log: str = None,
                    chunk: int = 64):
    """Write profiles/<entry>_<workload>.kernel_trace.txt from a rocprofv3
    --kernel-trace --stats CSV directory: the op kernel's duration statistics
    and launch resources, next to bench.py's own event time of the profiled
    run (run_log) and of an unprofiled run (plain_log), when given."""
    import csv
    import glob
    from chunked_gated_delta_token_amd import workloads as W
    if op == "chain":
        raise SystemExit("kernel traces are summarized per kernel: use --op fused, gate_cumsum, scaled_dot or solve_tril")
    key = op_key(op, chunk)
    kname = kernel_name(key, workload)
    stats = [r for path in glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
             for r in csv.DictReader(open(path, newline="")) if f"::{kname}<" in r["Name"]]
    if len(stats) != 1:
        raise SystemExit(f"expected one kernel matching {kname} in {directory}, found {len(stats)}")
    st = stats[0]
    disp, durations = None, []
    for path in glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(path, newline="")):
            if r["Kernel_Name"] == st["Name"]:
                disp = disp or r
                durations.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    durations = [d for _, d in sorted(durations)]
    w = W.WORKLOADS[workload]
    cu = W.generate(workload).cu_seqlens if w.n_seqs else None
    nbytes = algorithmic_bytes(w, w.B * w.T, op, cu, chunk)
    avg = float(st["AverageNs"])

    def event_us(log):
        if not log or not os.path.exists(log):
            return None
        for line in open(log):
            if line.startswith("{"):
                d = json.loads(line)
                return 1e3 * d["roofline"]["event_ms_per_step"]
        return None

    ev_prof, ev_plain = event_us(run_log), event_us(plain_log)
    sel = f"--op {op} --workload {workload}" + (f" --chunk {chunk}" if chunk != 64 else "")
    lines = [
        f"# rocprofv3 kernel trace: {kname}, workload {workload} ({w.B},{w.T},{w.H},{w.K}) "
        f"{w.in_dtype} -> {w.out_dtype}; {nbytes} algorithmic bytes per launch",
        "# commands (from /tmp, repository at $R; the last one wrote this file):",
        f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o kt -- python -u $R/bench.py {sel} "
        "--steps 200 --warmup 20 --no-cpu-baseline --no-second-target --no-floor > <run_log>",
        f"#   python -u $R/bench.py {sel} --no-cpu-baseline --no-second-target --no-floor > <plain_log>",
        f"#   python $R/bench.py --summarize-trace <dir> {sel} --run-log <run_log> --plain-log <plain_log>",
        f"kernel_source_sha256_16: {source_digest(op)}",
        f"kernel: {st['Name']}",
        f"calls: {st['Calls']}",
        f"average_ns: {avg:.1f}",
        f"min_ns: {st['MinNs']}",
        f"max_ns: {st['MaxNs']}",
        f"stddev_ns: {float(st['StdDev']):.1f}",
        f"share_of_gpu_time_percent: {st['Percentage']}",
    ]
    if disp is not None:
        lines += [f"grid_x: {disp['Grid_Size_X']}", f"workgroup_x: {disp['Workgroup_Size_X']}",
                  f"lds_bytes_per_workgroup: {disp['LDS_Block_Size']}  # static; one-wave-per-tile kernels add 5888 per wave at launch", f"scratch_bytes: {disp['Scratch_Size']}",
                  f"vgpr_count: {disp['VGPR_Count']}", f"sgpr_count: {disp['SGPR_Count']}"]
    lines.append(f"algorithmic_GBs_at_average: {nbytes / avg:.1f}")
    lines.append("# durations are device-side (dispatch start to end), eager warmup launches included")
    if len(durations) >= 200:
        import statistics
        last = durations[-200:]
        lines.append(f"median_ns: {statistics.median(durations):.1f}")
        q = statistics.quantiles(last, n=10)
        lines.append(f"timed_graph_replay_p10_ns: {q[0]:.1f}")
        lines.append(f"timed_graph_replay_median_ns: {statistics.median(last):.1f}")
        lines.append(f"timed_graph_replay_p90_ns: {q[-1]:.1f}")
        lines.append(f"timed_graph_replay_average_ns: {statistics.mean(last):.1f}  # the last 200 dispatches")
    if ev_prof is not None:
        lines.append(f"bench_event_us_per_step_under_profiler: {ev_prof:.3f}")
    if ev_plain is not None:
        lines.append(f"bench_event_us_per_step_unprofiled: {ev_plain:.3f}")
        lines.append(f"trace_average_vs_unprofiled_event: {avg / 1e3 / ev_plain - 1.0:+.3%}")
        if len(durations) >= 200:
            lines.append(f"timed_replay_average_vs_unprofiled_event: "
                         f"{statistics.mean(durations[-200:]) / 1e3 / ev_plain - 1.0:+.3%}")
    path = os.path.join(ROOT, "profiles", f"{ENTRY[key]}_{workload}.kernel_trace.txt")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measure(name: str, op: str, chunk: int, steps: int, warmup: int, timing: str = "graph", detail: bool = False):
    """Time `steps` steps of one op on one workload: inputs resident in HBM,
    R buffer sets rotated so that every step reads HBM, the steps captured in
    one HIP graph (timing "graph") and replayed once between two device
    synchronisations, HIP events recorded on the launch stream around the
    replay.  Returns the measured values and what they were measured on."""
    import numpy as np
    import torch
    from chunked_gated_delta_token_amd import kkt
    from chunked_gated_delta_token_amd import workloads as W

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
    if op == "gate_cumsum":
        if inp.g_raw is None:
            raise SystemExit(f"--op gate_cumsum needs a workload with a gate ({name} has none)")
        g0 = torch.from_numpy(inp.g_raw).to(dev)  # per-token log-decays, summed by the kernel
    if chunk != 64 and op not in ("fused", "gate_cumsum"):
        raise SystemExit("--chunk 128 applies to the fused op and its gate-sum form only")
    floor_fn = None
    if op == "floor":
        if inp.cu_seqlens is not None or w.T % 64:
            raise SystemExit("--op floor: sequences of whole 64-token chunks only")
        floor_fn = load_floor()
    nbytes = algorithmic_bytes(w, n_tokens, op, inp.cu_seqlens, chunk)
    num_seqs = 0 if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
    stream = torch.cuda.Stream(dev)
    shape = (w.B, w.T, w.H, 64)
    if op == "solve_tril":
        # the solve's input: A of the workload, made once by the first step
        A0 = torch.empty(shape, dtype=torch.float32, device=dev)
        st = lib.kkt_scaled_dot(k0.data_ptr(), None if g0 is None else g0.data_ptr(),
                                None if b0 is None else b0.data_ptr(), None if cu0 is None else cu0.data_ptr(),
                                num_seqs, w.B, w.T, w.H, w.K, 64, kdt[w.in_dtype], A0.data_ptr(), None)
        if st != 0:
            raise RuntimeError(f"kkt_scaled_dot status {st}: {kkt.last_error()}")
        torch.cuda.synchronize()
    # bytes one buffer set occupies (every tensor a step touches)
    a_bytes = int(np.prod(shape)) * 4
    out_bytes = int(np.prod(shape)) * ESIZE[w.out_dtype]
    set_bytes = {"fused": nbytes, "gate_cumsum": nbytes, "scaled_dot": nbytes, "chain": nbytes + a_bytes,
                 "solve_tril": a_bytes + out_bytes, "floor": nbytes}[op]
    R = max(2, -(-2 * MALL_BYTES // set_bytes))
    sets = []
    for _ in range(R):
        s_ = dict(cu=None if cu0 is None else cu0.clone())
        if op != "solve_tril":
            s_.update(k=k0.clone(), g=None if g0 is None else g0.clone(), b=None if b0 is None else b0.clone())
        if op in ("scaled_dot", "chain"):
            s_["A"] = torch.empty(shape, dtype=torch.float32, device=dev)
        if op == "solve_tril":
            s_["A"] = A0.clone()
        if op != "scaled_dot":
            s_["out"] = torch.empty(shape[:3] + (chunk,), dtype=tdt[w.out_dtype], device=dev)
        if op == "gate_cumsum":
            s_["g_out"] = torch.empty(shape[:3], dtype=torch.float32, device=dev)
        sets.append(s_)
    del k0, g0, b0
    if op == "solve_tril":
        del A0
    # the copies above ran on the current stream; the launches go to `stream`
    torch.cuda.synchronize()

    def ptr(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    sp = ctypes.c_void_p(stream.cuda_stream)

    def step_calls(s_):
        """(entry point, arguments) of the launches one step makes."""
        kargs = (ptr(s_.get("k")), ptr(s_.get("g")), ptr(s_.get("b")), ptr(s_["cu"]), num_seqs, w.B, w.T, w.H, w.K, 64,
                 kdt[w.in_dtype])
        if op == "fused":
            kargs_c = kargs[:9] + (chunk,) + kargs[10:]
            return [(lib.kkt_solve, kargs_c + (kdt[w.out_dtype], ptr(s_["out"]), sp))]
        if op == "gate_cumsum":
            kargs_c = kargs[:9] + (chunk,) + kargs[10:]
            return [(lib.kkt_solve_gate_cumsum, kargs_c + (kdt[w.out_dtype], ptr(s_["out"]), ptr(s_["g_out"]), sp))]
        if op == "floor":
            return [(floor_fn, (ptr(s_["k"]), ptr(s_.get("g")), ptr(s_.get("b")), w.B, w.T, w.H,
                                w.K * ESIZE[w.in_dtype], 64 * ESIZE[w.out_dtype], ptr(s_["out"]), sp))]
        tril = (lib.kkt_solve_tril, (ptr(s_["A"]), ptr(s_["cu"]), num_seqs, w.B, w.T, w.H, 64, kdt[w.out_dtype],
                                     ptr(s_.get("out")), sp))
        dot = (lib.kkt_scaled_dot, kargs + (ptr(s_["A"]), sp))
        return {"scaled_dot": [dot], "solve_tril": [tril], "chain": [dot, tril]}[op]

    calls = [step_calls(s_) for s_ in sets]

    def launch(i):
        for fn, a in calls[i % R]:
            st = fn(*a)
            if st != 0:
                raise RuntimeError(f"{fn.__name__} status {st}" + ("" if op == "floor" else f": {kkt.last_error()}"))

    # correctness guard on the bench inputs (cheap structural check, no oracle)
    with torch.cuda.stream(stream):
        launch(0)
    torch.cuda.synchronize()
    if op != "floor":  # (the reference's output is the key bytes)
        o = sets[0]["A" if op == "scaled_dot" else "out"].float()
        assert torch.isfinite(o).all().item(), "non-finite output"
        del o

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()

    K = steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph = None
    if timing == "graph":
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

    if detail:
        # per-launch event pairs (eager), for comparison with the profiler
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(64)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(64)]
        for i in range(64):
            starts[i].record(stream)
            launch(i)
            ends[i].record(stream)
        torch.cuda.synchronize()
        per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
        print(json.dumps({"workload": name, "per_launch_event_ms_median": per[len(per) // 2],
                          "per_launch_event_ms_min": per[0], "graph_event_ms": ev_ms, "wall_ms": ms_per_step}),
              file=sys.stderr, flush=True)
    del graph, sets, calls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    n_tiles = w.H * (sum(-(-(int(inp.cu_seqlens[s + 1]) - int(inp.cu_seqlens[s])) // chunk)
                         for s in range(num_seqs)) if num_seqs else w.B * (-(-w.T // chunk)))
    key = op_key(op, chunk)
    return {"inp": inp, "w": w, "nbytes": nbytes, "R": R, "ms_per_step": ms_per_step, "ev_ms": ev_ms,
            "n_tiles": n_tiles, "key": key,
            "kernel": KERNELS[key] if op == "chain" else kernel_name(key, name)}


# The second shape the target is quoted on (PR #135 performance table, row
# (2,16384,32,128)): timed beside the headline in the default run.
SECOND_TARGET = "B2_T16384_H32_bf16_bf16"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--op", choices=["fused", "gate_cumsum", "scaled_dot", "solve_tril", "chain", "floor"],
                    default="fused", help="what one step runs (default: the fused op; floor: the memory-traffic "
                                          "reference kernel)")
    ap.add_argument("--chunk", type=int, choices=[64, 128], default=64,
                    help="chunk size of the fused op (128: the 128-token variant)")
    ap.add_argument("--timing", choices=["graph", "eager"], default="graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-second-target", action="store_true",
                    help="time only the headline workload (by default the fused op's run also times "
                         "(2,16384,32,128) and reports it under second_target)")
    ap.add_argument("--no-floor", action="store_true",
                    help="skip the memory-traffic reference that the fused op's default run also times")
    ap.add_argument("--detail", action="store_true", help="also print per-launch event timings to stderr")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the op, run --steps plain device copies of BYTES bytes (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("OP_FETCH", "OP_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the HBM-traffic summary from four rocprofv3 --pmc output directories")
    ap.add_argument("--copy-bytes", type=int, default=0, help="size used by the copy-calibration runs")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the kernel-trace summary of --op from a rocprofv3 --kernel-trace --stats directory")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="write the MFMA-counter summary of --op from a rocprofv3 --pmc directory")
    ap.add_argument("--run-log", help="bench.py output of the profiled run (with --summarize-trace)")
    ap.add_argument("--plain-log", help="bench.py output of an unprofiled run (with --summarize-trace)")
    args = ap.parse_args()

    if args.summarize_mfma:
        from chunked_gated_delta_token_amd import workloads as W
        summarize_mfma(args.summarize_mfma, args.op, args.workload or W.BENCH_WORKLOAD, args.chunk)
        return

    if args.summarize_trace:
        from chunked_gated_delta_token_amd import workloads as W
        summarize_trace(args.summarize_trace, args.op, args.workload or W.BENCH_WORKLOAD, args.run_log,
                        args.plain_log, args.chunk)
        return

    if args.summarize_traffic:
        from chunked_gated_delta_token_amd import workloads as W
        summarize_traffic(args.summarize_traffic, args.copy_bytes, args.op, args.workload or W.BENCH_WORKLOAD,
                          args.chunk)
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

    from chunked_gated_delta_token_amd import workloads as W

    name = args.workload or W.BENCH_WORKLOAD
    op, chunk = args.op, args.chunk
    m = measure(name, op, chunk, args.steps, args.warmup, args.timing, args.detail)
    inp, w, nbytes, R = m["inp"], m["w"], m["nbytes"], m["R"]
    ms_per_step, ev_ms, n_tiles, key = m["ms_per_step"], m["ev_ms"], m["n_tiles"], m["key"]
    K = args.steps
    achieved = nbytes / (ev_ms * 1e-3) / 1e9
    digest = source_digest(op)
    traffic = None if op == "chain" else read_traffic(digest, traffic_file(key, name))
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    metric = METRIC if (op == "fused" and chunk == 64 and name == W.BENCH_WORKLOAD) else {
        "fused": f"fused KKT+solve{' with 128-token chunks' if chunk == 128 else ''} ms/iter & achieved HBM "
                 f"GB/s on {name}, 1 GPU",
        "gate_cumsum": f"fused KKT+solve{' with 128-token chunks' if chunk == 128 else ''} and the chunk-local gate "
                       f"sum in the kernel ms/iter & achieved HBM GB/s on {name}, 1 GPU",
        "scaled_dot": "KKT A alone (first step of the unfused chain) ms/iter & achieved HBM GB/s, 1 GPU",
        "solve_tril": "solve of a given A (second step of the unfused chain) ms/iter & achieved HBM GB/s, 1 GPU",
        "chain": "unfused two-step chain (A through HBM) ms/iter & GB/s of the fused op's bytes, 1 GPU",
        "floor": f"memory-traffic reference (the fused op's bytes and access pattern, no arithmetic) ms/iter & "
                 f"HBM GB/s on {name}, 1 GPU"}[op]
    pages_ms = {"fused": PAGES_FUSED_MS, "chain": PAGES_TWO_OP_MS}.get(op) if chunk == 64 else None
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(pages_ms / ms_per_step, 3) if (pages_ms and name == W.BENCH_WORKLOAD) else None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": name, "op": op, "chunk": chunk, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "in_dtype": w.in_dtype,
                   "out_dtype": w.out_dtype, "gate": w.gate, "beta": w.beta, "tiles": n_tiles,
                   "algorithmic_bytes": nbytes, "buffer_sets": R, "timing": args.timing,
                   "chunks_per_s": round(n_tiles / (ms_per_step * 1e-3), 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": m["kernel"],
                     "event_ms_per_step": round(ev_ms, 6), "launches_per_step": 2 if op == "chain" else 1,
                     "kernel_source_sha256_16": digest},
    }
    if op == "fused" and chunk == 64 and name == W.BENCH_WORKLOAD and not args.no_second_target:
        # the second shape of the target, timed the same way in the same run
        m2 = measure(SECOND_TARGET, "fused", 64, args.steps, min(args.warmup, 20), args.timing, args.detail)
        w2 = m2["w"]
        ach2 = m2["nbytes"] / (m2["ev_ms"] * 1e-3) / 1e9
        line["second_target"] = {
            "workload": SECOND_TARGET, "B": w2.B, "T": w2.T, "H": w2.H, "K": w2.K, "in_dtype": w2.in_dtype,
            "out_dtype": w2.out_dtype, "tiles": m2["n_tiles"], "algorithmic_bytes": m2["nbytes"],
            "buffer_sets": m2["R"], "steps": args.steps, "ms_per_step": round(m2["ms_per_step"], 6),
            "value": round(m2["nbytes"] / (m2["ms_per_step"] * 1e-3) / 1e9, 2), "unit": "GB/s",
            "event_ms_per_step": round(m2["ev_ms"], 6), "achieved": round(ach2, 2),
            "frac": round(ach2 / HBM_PEAK_GBS, 4), "kernel": m2["kernel"],
            "traffic": read_traffic(digest, traffic_file("fused", SECOND_TARGET)),
            "vs_baseline": round(PAGES_FUSED_MS_SECOND / m2["ms_per_step"], 3)}
    mf = None if op == "chain" else read_mfma(digest, mfma_file(key, name))
    if mf is not None:
        # matrix-core use of the step, from the committed counter summary and
        # this run's event time: busy share of all SIMD cycles, and the Gram's
        # (16-bit) MFMA rate against the dense bf16/f16 peak
        cycles = ev_ms * 1e-3 * CLOCK_HZ * N_SIMDS
        gram = mf["mfma_flop_bf16_per_launch"] + mf["mfma_flop_f16_per_launch"]
        line["roofline"]["mfma"] = {
            "busy_frac": round(mf["mfma_busy_cycles_per_launch"] / cycles, 4),
            "gram_tflops": round(gram / (ev_ms * 1e-3) / 1e12, 2) if gram else None,
            "gram_frac_of_16bit_peak": round(gram / (ev_ms * 1e-3) / 2.5e15, 4) if gram else None,
            "f32_tflops": round(mf["mfma_flop_f32_per_launch"] / (ev_ms * 1e-3) / 1e12, 2),
        }
    if op == "fused" and chunk == 64 and name == W.BENCH_WORKLOAD and not args.no_floor:
        # the memory-traffic reference on the same workloads, timed the same
        # way: what the same bytes in the same pattern take with no arithmetic
        for wl, obj in ((name, line["roofline"]), (SECOND_TARGET, line.get("second_target"))):
            if obj is None:
                continue
            mfl = measure(wl, "floor", 64, args.steps, min(args.warmup, 20), args.timing)
            achf = mfl["nbytes"] / (mfl["ev_ms"] * 1e-3) / 1e9
            obj["floor"] = {"kernel": mfl["kernel"], "event_ms_per_step": round(mfl["ev_ms"], 6),
                            "achieved": round(achf, 2), "frac": round(achf / HBM_PEAK_GBS, 4),
                            "kernel_source_sha256_16": source_digest("floor")}
    if not args.no_cpu_baseline and op != "floor":
        line["cpu_baseline"] = cpu_baseline(inp, nbytes, args.cpu_seconds, op, chunk)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
