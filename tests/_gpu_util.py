"""Helpers shared by the GPU test modules: moving seeded inputs to the
device and results back (test infrastructure)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from chunked_gated_delta_token_amd import workloads as W

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def say(msg):
    """Print and flush, so that a log names the case if a run ends early."""
    print(msg, flush=True)
    sys.stdout.flush()


def load_kkt():
    """The binding module, after checking for a gfx950 GPU and the built
    library (raises otherwise: there is no fallback)."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from chunked_gated_delta_token_amd import kkt as mod
    mod.load_library()
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name
    return mod


def to_device(inp: W.Inputs, dev="cuda:0"):
    dt = inp.workload.in_dtype
    if dt == "f32":
        k = torch.from_numpy(inp.k_store).to(dev)
    else:
        k = torch.from_numpy(inp.k_store.view(np.int16)).to(dev).view(TORCH_DT[dt])
    g = None if inp.g is None else torch.from_numpy(inp.g).to(dev)
    b = None if inp.beta is None else torch.from_numpy(inp.beta).to(dev)
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to(dev)
    return k, g, b, cu


def from_device(out: torch.Tensor, out_dtype: str) -> np.ndarray:
    if out_dtype == "f32":
        return out.cpu().numpy()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)
