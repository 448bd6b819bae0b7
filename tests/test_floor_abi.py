"""The memory-traffic reference library (libkkt_floor.so) on the CPU: it
exports exactly what include/kkt_floor.h declares, the header compiles as
C, and invalid arguments are rejected before any HIP call (nothing here
launches a kernel)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kkt_floor.h")
LIB = os.path.join(ROOT, "chunked_gated_delta_token_amd", "libkkt_floor.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def fn():
    if not os.path.exists(LIB):
        from chunked_gated_delta_token_amd import build
        build.build_floor()
    f = ctypes.CDLL(LIB).kkt_floor_copy
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    return f


def test_exports_what_the_header_declares(fn):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = set(re.findall(r"^\s*int\s+(kkt_\w+)\s*\(", text, flags=re.M))
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    assert set(re.findall(r"\s[TW]\s(kkt_\w+)$", out, flags=re.M)) == declared == {"kkt_floor_copy"}


GOOD = dict(k=16, g=None, b=None, B=1, T=64, H=1, krb=256, orb=256, out=16)


@pytest.mark.parametrize("over", [dict(k=None), dict(out=None), dict(B=0), dict(H=0), dict(T=0), dict(T=-64),
                                  dict(T=100), dict(krb=64), dict(krb=1024), dict(krb=192), dict(orb=64),
                                  dict(orb=512), dict(H=1 << 24), dict(B=1 << 40, T=1 << 20)])
def test_invalid_arguments_rejected(fn, over):
    a = dict(GOOD, **over)
    assert fn(a["k"], a["g"], a["b"], a["B"], a["T"], a["H"], a["krb"], a["orb"], a["out"], None) == 1


def test_header_compiles_as_c_and_links(tmp_path, fn):
    src = tmp_path / "t.c"
    src.write_text('#include "kkt_floor.h"\n#include <stdio.h>\n'
                   'int main(void){ int s = kkt_floor_copy(0,0,0,1,64,1,256,256,0,0); printf("%d\\n", s);'
                   ' return s == 1 ? 0 : 1; }\n')
    exe = tmp_path / "t"
    libdir = os.path.dirname(LIB)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    f"-I{ROCM}/include", str(src), "-o", str(exe), f"-L{libdir}", "-lkkt_floor",
                    f"-Wl,-rpath,{libdir}"], check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
