"""CPU sanitizer builds: AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (plain C) is built with both and every pin of
  tests/test_oracle_pins.py runs on that build, in a child process with the
  sanitizer runtime preloaded (Python itself is not instrumented).  A copy of
  the oracle with a planted out-of-bounds write must be stopped by it, which
  shows that the run really is checked.
* The library is built with both on its host pass (the device code as
  usual) and its host-side argument handling is exercised through the C ABI:
  every invalid-argument path of every entry point, T = 0 no-ops with every K,
  the options, the per-thread error text.  No call passes the checks with
  T > 0, so nothing is ever launched, also on a machine with a GPU.

Both children abort on the first sanitizer report; the tests also look for
report text in their output.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORT_MARKS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "UndefinedBehaviorSanitizer")


def _gcc_runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc has no {name}")
    return path


def _clang_asan_runtime() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        pytest.skip("no clang AddressSanitizer runtime under ROCm")
    return found[-1]


def _sanitizer_env(preload: str, **extra) -> dict:
    env = dict(os.environ)
    env.update(LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT, **extra)
    return env


def _assert_clean(res):
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    for mark in REPORT_MARKS:
        assert mark not in out, out[-4000:]


# ---------------------------------------------------------------- the oracle
@pytest.fixture(scope="module")
def sanitized_oracle(tmp_path_factory):
    import oracle
    return oracle.build(out=str(tmp_path_factory.mktemp("asan_oracle") / "libkkt_oracle_asan.so"), sanitize=True)


def test_oracle_pins_under_asan_and_ubsan(sanitized_oracle):
    env = _sanitizer_env(_gcc_runtime("libasan.so"), KKT_ORACLE_LIB=sanitized_oracle, OMP_NUM_THREADS="4")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                          "-q", "-x", "-p", "no:cacheprovider"], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=600)
    _assert_clean(res)
    assert " passed" in res.stdout, res.stdout[-2000:]


def test_planted_out_of_bounds_write_is_caught(tmp_path):
    """A copy of the oracle that writes one element past the end of its
    output: the sanitized build must abort with an AddressSanitizer report."""
    import oracle
    src = open(os.path.join(ROOT, "oracle", "kkt_oracle.c")).read()
    anchor = "int kkt_oracle_chunk_cumsum("
    assert anchor in src
    # the planted mistake: a helper called first thing writes out[total]
    plant = textwrap.dedent("""
        static void planted_write_past_end(double* out, int64_t n) { out[n] = 1.0; }
        """)
    body_start = src.index("{", src.index(anchor)) + 1
    mutated = src[:src.index(anchor)] + plant + src[src.index(anchor):body_start] + \
        "\n    planted_write_past_end(g_out, B * T * H);\n" + src[body_start:]
    path = tmp_path / "kkt_oracle_planted.c"
    path.write_text(mutated)
    lib = oracle.build(out=str(tmp_path / "libplanted.so"), src=str(path), sanitize=True)
    code = ("import numpy as np, oracle; "
            "oracle.chunk_cumsum_ref(np.ones((1, 5, 2)))")
    env = _sanitizer_env(_gcc_runtime("libasan.so"), KKT_ORACLE_LIB=lib)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                         timeout=120)
    assert res.returncode != 0
    assert "ERROR: AddressSanitizer: heap-buffer-overflow" in res.stderr, res.stderr[-3000:]


# ---------------------------------------------------------------- the library's host side
HOST_SANITIZERS = ("-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer")

# Runs in the child: every call either fails an argument check or has T = 0.
ABI_EXERCISE = r'''
import ctypes, sys, threading
lib = ctypes.CDLL(sys.argv[1])
lib.kkt_last_error.restype = ctypes.c_char_p
lib.kkt_get_option.restype = ctypes.c_int64
lib.kkt_set_option.argtypes = [ctypes.c_int, ctypes.c_int64]
lib.kkt_get_option.argtypes = [ctypes.c_int]
I = ctypes.c_int64
P = ctypes.c_void_p
F = dict(k=16, g=None, beta=None, cu=None, ns=0, B=1, T=64, H=1, K=128, ch=64, di=1, do=0, out=16)

def solve(**o):
    a = dict(F, **o)
    return lib.kkt_solve(P(a["k"]), P(a["g"]), P(a["beta"]), P(a["cu"]), I(a["ns"]), I(a["B"]), I(a["T"]),
                         I(a["H"]), I(a["K"]), I(a["ch"]), a["di"], a["do"], P(a["out"]), None)

def gsum(**o):
    a = dict(F, g=32)
    a.update(o)
    return lib.kkt_solve_gate_cumsum(P(a["k"]), P(a["g"]), P(a["beta"]), P(a["cu"]), I(a["ns"]), I(a["B"]),
                                     I(a["T"]), I(a["H"]), I(a["K"]), I(a["ch"]), a["di"], a["do"], P(a["out"]),
                                     P(a.get("gout")), None)

def sdot(**o):
    a = dict(F, **o)
    return lib.kkt_scaled_dot(P(a["k"]), P(a["g"]), P(a["beta"]), P(a["cu"]), I(a["ns"]), I(a["B"]), I(a["T"]),
                              I(a["H"]), I(a["K"]), I(a["ch"]), a["di"], P(a["out"]), None)

def tril(**o):
    a = dict(F, **o)
    return lib.kkt_solve_tril(P(a["k"]), P(a["cu"]), I(a["ns"]), I(a["B"]), I(a["T"]), I(a["H"]), I(a["ch"]),
                              a["do"], P(a["out"]), None)

bad = [dict(ch=32), dict(ch=256), dict(di=3), dict(do=-1), dict(B=0), dict(H=0), dict(T=-1), dict(K=100),
       dict(K=20), dict(K=6, di=0), dict(K=288), dict(K=0), dict(cu=16, ns=2, B=2), dict(cu=16, ns=0), dict(k=None), dict(out=None),
       dict(k=18), dict(out=72), dict(g=18), dict(beta=17), dict(cu=18, ns=1), dict(B=1 << 40, T=1 << 20)]
# the arguments each entry point reads: an override of any other argument
# would leave the call valid (and so launching), so it is not applied
reads = {solve: set(F), gsum: set(F), sdot: set(F) - {"do"}, tril: set(F) - {"g", "beta", "K", "di"}}
for fn in (solve, gsum, sdot, tril):
    for o in bad:
        if not set(o) <= reads[fn]:
            continue
        st = fn(**o)
        if st == 0:
            raise SystemExit(f"{fn.__name__}{o} passed its checks")
        assert lib.kkt_last_error()
assert gsum(g=None) == 1 and gsum(gout=18) == 1
for K in list(range(8, 257, 8)) + [4, 12, 36, 100, 252]:
    for di in ((0,) if K % 8 else (0, 1, 2)):
        for ch in (64, 128):
            assert solve(K=K, di=di, ch=ch, T=0) == 0, lib.kkt_last_error()
            assert gsum(K=K, di=di, ch=ch, T=0) == 0, lib.kkt_last_error()
        assert sdot(K=K, di=di, T=0) == 0, lib.kkt_last_error()
assert tril(T=0) == 0
assert solve(T=0, k=None, out=None) == 0
for v in (0, 1, 7, 1 << 40, -1):
    assert lib.kkt_set_option(0, v) == 0 and lib.kkt_get_option(0) == v
assert lib.kkt_set_option(0, -2) == 1 and lib.kkt_set_option(7, 0) == 1 and lib.kkt_get_option(7) == -1
assert lib.kkt_set_option(1, 3) == 0 and lib.kkt_get_option(1) == 1

errors = []
def worker(i):
    for r in range(200):
        st = solve(K=100 + 32 * (i % 2)) if i % 2 == 0 else sdot(ch=128)
        msg = lib.kkt_last_error().decode()
        want = "K must be" if i % 2 == 0 else "chunk_size"
        if st == 0 or want not in msg:
            errors.append((i, r, st, msg))
        lib.kkt_set_option(0, r)
threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
[t.start() for t in threads]
[t.join() for t in threads]
assert not errors, errors[:3]
assert lib.kkt_version() == 904
print("abi exercise ok")
'''


def test_library_host_side_under_asan_and_ubsan(tmp_path):
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present: the host-side exercise runs only where no call can reach one")
    from chunked_gated_delta_token_amd import build
    lib = build.build(extra_flags=HOST_SANITIZERS, out=str(tmp_path / "libkkt_solve_asan.so"))
    env = _sanitizer_env(_clang_asan_runtime())
    res = subprocess.run([sys.executable, "-c", ABI_EXERCISE, lib], capture_output=True, text=True, env=env,
                         cwd=str(tmp_path), timeout=600)
    _assert_clean(res)
    assert "abi exercise ok" in res.stdout
