"""GPU check of the memory-traffic reference (libkkt_floor.so): every byte
of the output is the key byte the header names (16-byte piece c of an output
row is piece c mod (key row bytes / 16) of the same key row), for each
supported pair of row widths, with and without g and beta."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

from tests._gpu_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "chunked_gated_delta_token_amd", "libkkt_floor.so")


@pytest.fixture(scope="module")
def fn():
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is missing: build it with `python -m chunked_gated_delta_token_amd.build`")
    f = ctypes.CDLL(LIB).kkt_floor_copy
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    return f


@pytest.mark.parametrize("krb,orb", [(128, 128), (128, 256), (256, 128), (256, 256), (512, 128), (512, 256)])
@pytest.mark.parametrize("with_gb", [False, True])
def test_floor_copy_bytes(fn, krb, orb, with_gb):
    B, T, H = 2, 192, 3
    say(f"[case] floor copy krb={krb} orb={orb} g/beta={with_gb} B={B} T={T} H={H}")
    rng = np.random.default_rng(krb * 7 + orb + int(with_gb))
    k = rng.integers(0, 256, size=(B, T, H, krb), dtype=np.uint8)
    dev = torch.device("cuda:0")
    kd = torch.from_numpy(k).to(dev)
    out = torch.full((B, T, H, orb), 0xAB, dtype=torch.uint8, device=dev)
    g = torch.randn(B, T, H, device=dev) if with_gb else None
    b = torch.rand(B, T, H, device=dev) if with_gb else None
    st = fn(kd.data_ptr(), None if g is None else g.data_ptr(), None if b is None else b.data_ptr(), B, T, H, krb,
            orb, out.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(B, T, H, orb // 16, 16)
    pieces = k.reshape(B, T, H, krb // 16, 16)
    want = pieces[:, :, :, np.arange(orb // 16) % (krb // 16), :]
    assert np.array_equal(got, want)
