"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects invalid arguments before making any HIP call (so these
tests run without a GPU; nothing here launches a kernel)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kkt_solve.h")
LIB = os.path.join(ROOT, "chunked_gated_delta_token_amd", "libkkt_solve.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from chunked_gated_delta_token_amd import build
        build.build()
    from chunked_gated_delta_token_amd import kkt
    return kkt.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(kkt_[a-z_]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["kkt_get_option", "kkt_last_error", "kkt_scaled_dot", "kkt_set_option",
                                    "kkt_solve", "kkt_solve_gate_cumsum", "kkt_solve_tril", "kkt_version"]


def test_every_declared_symbol_is_exported(lib):
    from chunked_gated_delta_token_amd import kkt
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in kkt.SIGNATURES, name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s(kkt_\w+)$", out, flags=re.M))
    assert exported == set(declared_functions()), exported


def test_version(lib):
    assert lib.kkt_version() == 904


def _call(lib, **over):
    args = dict(k=16, g=None, beta=None, cu=None, num_seqs=0, B=1, T=64, H=1, K=128, chunk_size=64,
                in_dtype=1, out_dtype=0, out=16, stream=None)
    args.update(over)
    return lib.kkt_solve(args["k"], args["g"], args["beta"], args["cu"], args["num_seqs"], args["B"],
                         args["T"], args["H"], args["K"], args["chunk_size"], args["in_dtype"],
                         args["out_dtype"], args["out"], args["stream"])


@pytest.mark.parametrize("over,status,msg", [
    (dict(chunk_size=32), 2, "chunk_size"),
    (dict(chunk_size=256), 2, "chunk_size"),
    (dict(in_dtype=3), 1, "dtype"),
    (dict(out_dtype=-1), 1, "dtype"),
    (dict(B=0), 1, ">= 1"),
    (dict(H=0), 1, ">= 1"),
    (dict(T=-1), 1, ">= 1"),
    (dict(K=100), 2, "K must be"),
    (dict(K=20), 2, "K must be"),
    (dict(K=6, in_dtype=0), 2, "K must be"),
    (dict(K=258, in_dtype=0), 2, "K must be"),
    (dict(K=264), 2, "K must be"),
    (dict(K=288), 2, "K must be"),
    (dict(K=512), 2, "K must be"),
    (dict(K=0), 1, ">= 1"),
    (dict(cu=1, num_seqs=2, B=2), 1, "cu_seqlens"),
    (dict(cu=1, num_seqs=0), 1, "cu_seqlens"),
    (dict(k=None), 1, "NULL"),
    (dict(out=None), 1, "NULL"),
    (dict(k=16 + 2), 1, "16-byte aligned"),
    (dict(out=64 + 8), 1, "16-byte aligned"),
    (dict(g=16 + 2), 1, "4-byte aligned"),
    (dict(beta=16 + 1), 1, "4-byte aligned"),
    (dict(cu=16 + 2, num_seqs=1), 1, "4-byte aligned"),
    # T and the addresses travel in the kernels' preloaded 32-bit and 48-bit fields
    (dict(T=2 ** 32), 2, "below 2^32"),
    (dict(k=1 << 48), 2, "below 2^48"),
    (dict(out=(1 << 63) + 16), 2, "below 2^48"),
    (dict(g=1 << 48), 2, "below 2^48"),
    (dict(beta=(1 << 52) + 4), 2, "below 2^48"),
])
def test_invalid_arguments_rejected_on_host(lib, over, status, msg):
    from chunked_gated_delta_token_amd import kkt
    assert _call(lib, **over) == status
    assert msg in kkt.last_error()


@pytest.mark.parametrize("in_dtype", [0, 1, 2])
def test_k_check_takes_rows_of_whole_16_byte_pieces(lib, in_dtype):
    """Every K from 1 to 300: the call passes the argument checks exactly when
    K <= 256 and K * element size is a multiple of 16 bytes (fp32 keys: K a
    multiple of 4; bf16 / f16: of 8).  With T = 0 a passing call returns
    KKT_OK without launching anything (so this never touches a GPU, even
    where one is present)."""
    from chunked_gated_delta_token_amd import kkt
    size = 4 if in_dtype == 0 else 2
    for K in range(1, 301):
        want = kkt.KKT_OK if (K <= 256 and (K * size) % 16 == 0) else kkt.KKT_ERR_UNSUPPORTED
        for chunk in (64, 128):
            assert _call(lib, K=K, in_dtype=in_dtype, T=0, chunk_size=chunk) == want, (K, kkt.last_error())
        assert _call_scaled_dot(lib, K=K, in_dtype=in_dtype, T=0) == want, (K, kkt.last_error())


def test_options_round_trip_and_reject_bad_values(lib):
    """kkt_set_option / kkt_get_option: values round-trip (-1: the library's
    own choice, the default), an unknown option or a two-wave bound below -1
    is rejected and leaves the option as it was; the Python context manager
    restores the previous value."""
    from chunked_gated_delta_token_amd import kkt
    split0 = kkt.get_option(kkt.KKT_OPTION_SPLIT_MAX_TILES)
    val0 = kkt.get_option(kkt.KKT_OPTION_VALIDATE_CU_SEQLENS)
    assert split0 == int(os.environ.get("KKT_SPLIT_TILES") or -1)
    try:
        kkt.set_option(kkt.KKT_OPTION_SPLIT_MAX_TILES, 7)
        assert kkt.get_option(kkt.KKT_OPTION_SPLIT_MAX_TILES) == 7
        with pytest.raises(kkt.KKTInvalidArgument):
            kkt.set_option(kkt.KKT_OPTION_SPLIT_MAX_TILES, -2)
        assert kkt.get_option(kkt.KKT_OPTION_SPLIT_MAX_TILES) == 7
        with kkt.option(kkt.KKT_OPTION_SPLIT_MAX_TILES, -1):
            assert kkt.get_option(kkt.KKT_OPTION_SPLIT_MAX_TILES) == -1
        with kkt.option(kkt.KKT_OPTION_SPLIT_MAX_TILES, 0):
            assert kkt.get_option(kkt.KKT_OPTION_SPLIT_MAX_TILES) == 0
        assert kkt.get_option(kkt.KKT_OPTION_SPLIT_MAX_TILES) == 7
        kkt.set_option(kkt.KKT_OPTION_VALIDATE_CU_SEQLENS, 5)
        assert kkt.get_option(kkt.KKT_OPTION_VALIDATE_CU_SEQLENS) == 1
        assert lib.kkt_set_option(9, 1) == kkt.KKT_ERR_INVALID_ARGUMENT
        assert "unknown option" in kkt.last_error()
        assert lib.kkt_get_option(9) == -1
    finally:
        kkt.set_option(kkt.KKT_OPTION_SPLIT_MAX_TILES, split0)
        kkt.set_option(kkt.KKT_OPTION_VALIDATE_CU_SEQLENS, val0)


def test_options_start_from_the_environment(tmp_path):
    """The start values come from KKT_SPLIT_TILES and KKT_VALIDATE, read when
    the library is loaded (a fresh process here)."""
    code = ("import ctypes, sys; lib = ctypes.CDLL(sys.argv[1]); lib.kkt_get_option.restype = ctypes.c_int64; "
            "print(lib.kkt_get_option(0), lib.kkt_get_option(1))")
    env = dict(os.environ, KKT_SPLIT_TILES="33", KKT_VALIDATE="1")
    out = subprocess.run(["python3", "-c", code, LIB], capture_output=True, text=True, env=env, check=True)
    assert out.stdout.split() == ["33", "1"]
    env = {k: v for k, v in os.environ.items() if k not in ("KKT_SPLIT_TILES", "KKT_VALIDATE")}
    out = subprocess.run(["python3", "-c", code, LIB], capture_output=True, text=True, env=env, check=True)
    assert out.stdout.split() == ["-1", "0"]


def _call_scaled_dot(lib, **over):
    args = dict(k=16, g=None, beta=None, cu=None, num_seqs=0, B=1, T=64, H=1, K=128, chunk_size=64,
                in_dtype=1, A=16, stream=None)
    args.update(over)
    return lib.kkt_scaled_dot(args["k"], args["g"], args["beta"], args["cu"], args["num_seqs"], args["B"],
                              args["T"], args["H"], args["K"], args["chunk_size"], args["in_dtype"], args["A"],
                              args["stream"])


@pytest.mark.parametrize("over,status,msg", [
    (dict(chunk_size=128), 2, "chunk_size"),
    (dict(in_dtype=5), 1, "dtype"),
    (dict(H=0), 1, ">= 1"),
    (dict(K=84), 2, "K must be"),
    (dict(cu=16, num_seqs=1, B=3), 1, "cu_seqlens"),
    (dict(k=None), 1, "NULL"),
    (dict(A=None), 1, "NULL"),
    (dict(A=16 + 4), 1, "16-byte aligned"),
    (dict(g=16 + 2), 1, "4-byte aligned"),
])
def test_scaled_dot_invalid_arguments(lib, over, status, msg):
    from chunked_gated_delta_token_amd import kkt
    assert _call_scaled_dot(lib, **over) == status
    assert msg in kkt.last_error()


def test_chunk128_is_served_by_the_fused_entry_points_only(lib):
    """chunk_size 128 passes the argument checks of kkt_solve and
    kkt_solve_gate_cumsum (NULL pointers are then the first error) and is
    rejected by the two split steps."""
    from chunked_gated_delta_token_amd import kkt
    assert _call(lib, chunk_size=128, k=None) == 1 and "NULL" in kkt.last_error()
    assert _call_gate_cumsum(lib, chunk_size=128, k=None) == 1 and "NULL" in kkt.last_error()
    assert _call_scaled_dot(lib, chunk_size=128) == 2 and "chunk_size" in kkt.last_error()
    assert _call_solve_tril(lib, chunk_size=128) == 2 and "chunk_size" in kkt.last_error()


def _call_gate_cumsum(lib, **over):
    args = dict(k=16, g=32, beta=None, cu=None, num_seqs=0, B=1, T=64, H=1, K=128, chunk_size=64,
                in_dtype=1, out_dtype=0, out=16, g_out=None, stream=None)
    args.update(over)
    return lib.kkt_solve_gate_cumsum(args["k"], args["g"], args["beta"], args["cu"], args["num_seqs"], args["B"],
                                     args["T"], args["H"], args["K"], args["chunk_size"], args["in_dtype"],
                                     args["out_dtype"], args["out"], args["g_out"], args["stream"])


@pytest.mark.parametrize("over,status,msg", [
    (dict(chunk_size=32), 2, "chunk_size"),
    (dict(chunk_size=256), 2, "chunk_size"),
    (dict(out_dtype=9), 1, "dtype"),
    (dict(K=52), 2, "K must be"),
    (dict(T=-1), 1, ">= 1"),
    (dict(g=None), 1, "g_decay"),
    (dict(k=None), 1, "NULL"),
    (dict(out=16 + 4), 1, "16-byte aligned"),
    (dict(g=32 + 2), 1, "4-byte aligned"),
    (dict(g_out=64 + 1), 1, "4-byte aligned"),
    (dict(g_out=1 << 48), 2, "below 2^48"),
    (dict(g=(1 << 49) + 4), 2, "below 2^48"),
])
def test_gate_cumsum_invalid_arguments(lib, over, status, msg):
    from chunked_gated_delta_token_amd import kkt
    assert _call_gate_cumsum(lib, **over) == status
    assert msg in kkt.last_error()


def _call_solve_tril(lib, **over):
    args = dict(A=16, cu=None, num_seqs=0, B=1, T=64, H=1, chunk_size=64, out_dtype=0, out=16, stream=None)
    args.update(over)
    return lib.kkt_solve_tril(args["A"], args["cu"], args["num_seqs"], args["B"], args["T"], args["H"],
                              args["chunk_size"], args["out_dtype"], args["out"], args["stream"])


@pytest.mark.parametrize("over,status,msg", [
    (dict(chunk_size=16), 2, "chunk_size"),
    (dict(out_dtype=7), 1, "dtype"),
    (dict(B=0), 1, ">= 1"),
    (dict(T=-5), 1, ">= 1"),
    (dict(cu=16, num_seqs=0), 1, "cu_seqlens"),
    (dict(A=None), 1, "NULL"),
    (dict(out=None), 1, "NULL"),
    (dict(A=16 + 8), 1, "16-byte aligned"),
    (dict(cu=16 + 1, num_seqs=1), 1, "4-byte aligned"),
    (dict(T=2 ** 32 + 64), 2, "below 2^32"),
    (dict(out=1 << 48), 2, "below 2^48"),
])
def test_solve_tril_invalid_arguments(lib, over, status, msg):
    from chunked_gated_delta_token_amd import kkt
    assert _call_solve_tril(lib, **over) == status
    assert msg in kkt.last_error()


def test_split_entry_points_empty_is_a_no_op(lib):
    from chunked_gated_delta_token_amd import kkt
    assert _call_scaled_dot(lib, T=0, k=None, A=None) == 0
    assert kkt.last_error() == ""
    assert _call_solve_tril(lib, T=0, A=None, out=None) == 0
    assert kkt.last_error() == ""
    assert _call_gate_cumsum(lib, T=0, k=None, g=None, out=None) == 0
    assert kkt.last_error() == ""


def test_last_error_is_per_thread(lib):
    """Concurrent failing calls on several host threads: each thread reads
    its own message (argument checks only; no GPU needed)."""
    import threading
    from chunked_gated_delta_token_amd import kkt
    cases = [(dict(chunk_size=32), "chunk_size"), (dict(K=100), "K must be"), (dict(in_dtype=9), "dtype"),
             (dict(B=0), ">= 1")]
    errors = []

    def worker(over, msg):
        for _ in range(200):
            st = _call(lib, **over)
            text = kkt.last_error()
            if st == 0 or msg not in text:
                errors.append((over, st, text))
                return

    threads = [threading.Thread(target=worker, args=c) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_empty_sequence_is_a_no_op(lib):
    from chunked_gated_delta_token_amd import kkt
    assert _call(lib, T=0, k=None, out=None) == 0
    assert kkt.last_error() == ""


def test_python_binding_rejects_chunk_size():
    import torch
    from chunked_gated_delta_token_amd import kkt
    with pytest.raises(ValueError):
        kkt.kkt_solve(torch.zeros(1, 4, 1, 128), chunk_size=32)
    with pytest.raises(ValueError):
        kkt.kkt_scaled_dot(torch.zeros(1, 4, 1, 128), chunk_size=128)
    with pytest.raises(ValueError):
        kkt.kkt_solve_tril(torch.zeros(1, 4, 1, 64), chunk_size=16)
    with pytest.raises(ValueError):  # host tensor: no CPU fallback
        kkt.kkt_solve_tril(torch.zeros(1, 4, 1, 64))


def test_python_exceptions_follow_the_status(lib):
    """The binding raises ValueError for KKT_ERR_INVALID_ARGUMENT and
    NotImplementedError for KKT_ERR_UNSUPPORTED (both also KKTError, with the
    status and the library's message)."""
    from chunked_gated_delta_token_amd import kkt
    for over, cls, base in ((dict(B=0), kkt.KKTInvalidArgument, ValueError),
                            (dict(K=100), kkt.KKTUnsupported, NotImplementedError)):
        st = _call(lib, **over)
        err = kkt._error(st)
        assert type(err) is cls and isinstance(err, base) and isinstance(err, kkt.KKTError)
        assert err.status == st and kkt.last_error() in str(err)
    assert type(kkt._error(kkt.KKT_ERR_HIP)) is kkt.KKTError


def test_header_compiles_as_c_and_links(tmp_path, lib):
    """A plain C program includes the header, links the library and makes a
    host-only call (argument rejection)."""
    src = tmp_path / "t.c"
    src.write_text('#include "kkt_solve.h"\n#include <stdio.h>\n'
                   'int main(void){ kkt_status_t s = kkt_solve(0,0,0,0,0,1,64,1,128,32,KKT_DTYPE_BF16,'
                   'KKT_DTYPE_F32,0,0); printf("%d %d %s\\n", (int)s, kkt_version(), kkt_last_error());'
                   ' return s == KKT_ERR_UNSUPPORTED ? 0 : 1; }\n')
    exe = tmp_path / "t"
    libdir = os.path.dirname(LIB)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    f"-I{ROCM}/include", str(src), "-o", str(exe), f"-L{libdir}", "-lkkt_solve",
                    f"-Wl,-rpath,{libdir}"], check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "chunk_size must be 64" in res.stdout
