"""Compile the HIP library ``libkkt_solve.so`` for gfx950, in-tree.

    python -m chunked_gated_delta_token_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "kkt_solve.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkkt_solve.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, extra_flags=(), out: str = None) -> str:
    """Build the shared library (at ``out``, default the package's
    ``libkkt_solve.so``); returns its path.  Raises on failure."""
    lib = out or LIB
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU ops stay off (see the kernel notes); hipcc's host
           # pass warns that it does not know the feature, which is harmless
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA results in ordinary VGPRs: no accumulator-register copies
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wall", "-I", INCLUDE, "-o", lib + ".tmp", SRC, *extra_flags]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in res.stderr.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError("HIP build failed:\n" + res.stdout + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
