"""GPU: the C ABI driven from a plain C program (tests/c/abi_consumer.c),
with no Python binding and no torch in that process: HIP runtime calls for
memory and a stream, then kkt_solve, kkt_scaled_dot + kkt_solve_tril and an
in-place kkt_solve_gate_cumsum.  The inputs come from the seeded generator;
the results are checked here against the fp64 oracle (test infrastructure)."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from chunked_gated_delta_token_amd import workloads as W
from tests._compare import GATE_BOUND_ULPS, compare
from tests._gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "chunked_gated_delta_token_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def consumer(tmp_path_factory):
    assert os.path.exists(os.path.join(LIBDIR, "libkkt_solve.so")), "build the library first"
    exe = str(tmp_path_factory.mktemp("c_abi") / "abi_consumer")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    f"-I{ROCM}/include", os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-o", exe,
                    f"-L{LIBDIR}", "-lkkt_solve", f"-L{ROCM}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib"], check=True, capture_output=True)
    return exe


@pytest.mark.parametrize("B,T,H", [(1, 1000, 4), (1, 8192, 8)])
def test_c_program_drives_the_abi(consumer, tmp_path, B, T, H):
    """64 tiles (two-wave form) and 1024 tiles (one wave per tile)."""
    inp = W.generate("T256_H8_bf16_f32", B=B, T=T, H=H, seed=4900 + T)
    say(f"[case] C consumer of the ABI: B={B} T={T} H={H} K=128 bf16 -> f32")
    inp.k_store.astype(np.uint16).tofile(tmp_path / "k.bin")
    inp.g.astype(np.float32).tofile(tmp_path / "g.bin")
    inp.beta.astype(np.float32).tofile(tmp_path / "beta.bin")
    inp.g_raw.astype(np.float32).tofile(tmp_path / "g_raw.bin")
    res = subprocess.run([consumer, str(tmp_path), str(B), str(T), str(H), "128"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    shape = (B, T, H, 64)
    fused = np.fromfile(tmp_path / "x_fused.bin", dtype=np.float32).reshape(shape)
    chain = np.fromfile(tmp_path / "x_chain.bin", dtype=np.float32).reshape(shape)
    gsum_x = np.fromfile(tmp_path / "x_gsum.bin", dtype=np.float32).reshape(shape)
    g_sum = np.fromfile(tmp_path / "g_sum.bin", dtype=np.float32).reshape(shape[:3])
    assert np.array_equal(fused.view(np.uint32), chain.view(np.uint32))
    compare(fused, oracle.kkt_solve_ref(inp.k64(), inp.g, inp.beta, None), "f32", None, "C consumer, fused")
    # the in-place gate sum, against the oracle only (no value the library
    # wrote enters the reference): the summed gate within GATE_BOUND_ULPS
    # 2^-24 of the running sum of |decay| (the bar of the gate-sum tests),
    # the rows by the fused op's criteria against the oracle fed the decays
    X_ref, g_ref = oracle.kkt_solve_gate_cumsum_ref(inp.k64(), inp.g_raw, inp.beta, None)
    prefix_abs = oracle.chunk_cumsum_ref(np.abs(inp.g_raw.astype(np.float64)))
    bound = GATE_BOUND_ULPS * 2.0 ** -24 * prefix_abs
    err = np.abs(g_sum.astype(np.float64) - g_ref)
    assert not np.any(np.isnan(g_sum))
    assert np.all(err <= bound), f"gate sum error {float(np.max(err / np.maximum(bound, 1e-300))):.2f} x bound"
    compare(gsum_x, X_ref, "f32", None, "C consumer, gate sum")
    say("[ok] " + res.stdout.strip())
