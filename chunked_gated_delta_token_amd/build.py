"""Compile the HIP libraries for gfx950, in-tree: ``libkkt_solve.so`` (the
operation) and ``libkkt_floor.so`` (the memory-traffic reference the
benchmark times beside it).

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
FLOOR_SRC = os.path.join(PKG, "csrc", "stream_floor.hip")
FLOOR_LIB = os.path.join(PKG, "libkkt_floor.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, extra_flags=(), out: str = None, src: str = None) -> str:
    """Build the shared library of ``src`` (default the operation's source)
    at ``out`` (default the package's ``libkkt_solve.so``); returns its path.
    Raises on failure."""
    lib = out or LIB
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU ops stay off (see the kernel notes); hipcc's host
           # pass warns that it does not know the feature, which is harmless
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA results in ordinary VGPRs: no accumulator-register copies
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           # the leading scalar kernel arguments arrive in SGPRs at wave launch
           # (9 arguments, 14 dwords: the most the user SGPRs hold here)
           "-mllvm", "-amdgpu-kernarg-preload-count=9",
           "-Wall", "-I", INCLUDE, "-o", lib + ".tmp", src or SRC, *extra_flags]
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


def build_floor(verbose: bool = False) -> str:
    """Build ``libkkt_floor.so``, the memory-traffic reference; returns its path."""
    return build(verbose=verbose, out=FLOOR_LIB, src=FLOOR_SRC)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_floor(verbose=True))
