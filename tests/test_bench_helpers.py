"""bench.py's host-side helpers on the CPU: algorithmic bytes against the
workload table, and the summaries it writes from rocprofv3 CSV files (fed
here with small synthetic CSV files)."""
from __future__ import annotations

import csv
import os

import pytest

import bench
from chunked_gated_delta_token_amd import workloads as W

# per-workload algorithmic bytes of the fused op: k once, g and beta once, the
# output once (the workload table of the design notes)
FUSED_BYTES = {
    "T256_H8_bf16_f32": 1_064_960,
    "T2000_H8_bf16_bf16": 6_272_000,
    "T8192_H8_bf16_f32": 34_078_720,
    "B2_T16384_H32_bf16_bf16": 411_041_792,
    "varlen12_T16384_H7_f32_f32": 88_080_384,
}


@pytest.mark.parametrize("name", list(FUSED_BYTES))
def test_fused_algorithmic_bytes(name):
    w = W.WORKLOADS[name]
    assert bench.algorithmic_bytes(w, w.B * w.T, "fused") == FUSED_BYTES[name]
    assert bench.algorithmic_bytes(w, w.B * w.T, "chain") == FUSED_BYTES[name]


def test_other_ops_bytes():
    w = W.WORKLOADS["T8192_H8_bf16_f32"]
    n = w.B * w.T
    out = n * w.H * 64 * 4
    k = n * w.H * w.K * 2
    gb = n * w.H * 8
    assert bench.algorithmic_bytes(w, n, "scaled_dot") == k + gb + n * w.H * 64 * 4
    assert bench.algorithmic_bytes(w, n, "gate_cumsum") == k + gb + out + n * w.H * 4
    # 128 full chunks per head: 64*63/2 strictly lower fp32 entries each
    assert bench.algorithmic_bytes(w, n, "solve_tril") == 128 * w.H * 2016 * 4 + out
    assert bench.algorithmic_bytes(w, n, "fused", chunk=128) == k + gb + 2 * out


def test_chunk_lengths():
    w = W.WORKLOADS["T2000_H8_bf16_bf16"]
    assert bench.chunk_lengths(w, None) == [64] * 31 + [16]
    assert bench.chunk_lengths(w, [0, 70, 70, 200]) == [64, 6, 64, 64, 2]


def _write_csv(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=fields)
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE medians of the op, scaled by bytes per KiB of a
    copy of known size; the written file is read back only for the same
    kernel source."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    kn = "void (anonymous namespace)::kkt_solve_kernel<...>(KernelArgs)"
    dirs = [str(tmp_path / d) for d in ("of", "ow", "cf", "cw")]
    _write_csv(os.path.join(dirs[0], "x", "p_counter_collection.csv"),
               [{"Kernel_Name": kn, "Counter_Name": "FETCH_SIZE", "Counter_Value": v} for v in (100, 101, 102)], fields)
    _write_csv(os.path.join(dirs[1], "x", "p_counter_collection.csv"),
               [{"Kernel_Name": kn, "Counter_Name": "WRITE_SIZE", "Counter_Value": 50}], fields)
    _write_csv(os.path.join(dirs[2], "x", "p_counter_collection.csv"),
               [{"Kernel_Name": "copy_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": 8}], fields)
    _write_csv(os.path.join(dirs[3], "x", "p_counter_collection.csv"),
               [{"Kernel_Name": "copy_kernel", "Counter_Name": "WRITE_SIZE", "Counter_Value": 16}], fields)
    bench.summarize_traffic(dirs, 16384, "fused", "T8192_H8_bf16_f32")
    path = bench.traffic_file("fused", "T8192_H8_bf16_f32")
    assert os.path.exists(path)
    # fetch: median 101 KiB * (16384 B / 8 KiB) ; write: 50 KiB * (16384 B / 16 KiB)
    expected = 101 * 2048 + 50 * 1024
    assert bench.read_traffic(bench.source_digest(), path) == pytest.approx(expected, abs=1)
    assert bench.read_traffic("0000000000000000", path) is None


def test_gpus_above_one_exit_with_a_message(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_kernel_name_follows_the_launch_form(monkeypatch):
    """Small fused grids name the two-wave kernel, the rest one wave per tile,
    and so do the 16-bit-key, 16-bit-output fused grids; KKT_SPLIT_TILES
    sets one bound for all, as it does in the library (-1: its own choice)."""
    monkeypatch.delenv("KKT_SPLIT_TILES", raising=False)
    assert bench.kernel_name("fused", "T256_H8_bf16_f32") == "kkt_solve_split_kernel"      # 32 tiles
    assert bench.kernel_name("fused", "T2000_H8_bf16_bf16") == "kkt_solve_kernel"          # 256 tiles, 16-bit
    assert bench.kernel_name("fused", "T8192_H8_bf16_f32") == "kkt_solve_kernel"           # 1024 tiles
    assert bench.kernel_name("fused", "varlen12_T16384_H7_f32_f32") == "kkt_solve_kernel"  # 7 * (256 + 12)
    assert bench.kernel_name("fused128", "T256_H8_bf16_f32") == "kkt_solve128_kernel"
    assert bench.kernel_name("gate_cumsum", "T256_H8_bf16_f32") == "kkt_solve_gate_cumsum_split_kernel"
    assert bench.kernel_name("gate_cumsum", "T8192_H8_bf16_f32") == "kkt_solve_gate_cumsum_kernel"
    assert bench.kernel_name("gate_cumsum128", "T256_H8_bf16_f32") == "kkt_solve128_kernel"
    assert bench.kernel_name("solve_tril", "T2000_H8_bf16_bf16") == "kkt_solve_tril_split_kernel"
    assert bench.kernel_name("gate_cumsum", "T2000_H8_bf16_bf16") == "kkt_solve_gate_cumsum_split_kernel"
    assert bench.kernel_name("solve_tril", "T8192_H8_bf16_f32") == "kkt_solve_tril_kernel"
    assert bench.kernel_name("scaled_dot", "T256_H8_bf16_f32") == "kkt_scaled_dot_kernel"
    monkeypatch.setenv("KKT_SPLIT_TILES", "0")
    assert bench.kernel_name("fused", "T256_H8_bf16_f32") == "kkt_solve_kernel"
    monkeypatch.setenv("KKT_SPLIT_TILES", "256")
    assert bench.kernel_name("fused", "T2000_H8_bf16_bf16") == "kkt_solve_split_kernel"
    monkeypatch.setenv("KKT_SPLIT_TILES", "-1")
    assert bench.kernel_name("fused", "T2000_H8_bf16_bf16") == "kkt_solve_kernel"
    assert bench.kernel_name("fused", "T256_H8_bf16_f32") == "kkt_solve_split_kernel"
    monkeypatch.setenv("KKT_SPLIT_TILES", "1024")
    assert bench.kernel_name("fused", "T8192_H8_bf16_f32") == "kkt_solve_split_kernel"
