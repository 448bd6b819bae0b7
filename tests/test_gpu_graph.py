"""Every entry point captured in a HIP graph: the library launches kernels
only (no memset, no allocation), so replays, with eager work and
synchronisations between them, equal the eager result bit for bit, also
after the captured input buffers receive new values in place.  Covers the
128-token kernel (workgroup barriers, shared key image) and packed
sequences (offsets read in the kernel)."""
from __future__ import annotations

import pytest

from chunked_gated_delta_token_amd import workloads as W
from tests._gpu_util import load_kkt, say, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kkt():
    return load_kkt()


def _calls(kkt, name, k, g, b, cu):
    """(outputs, launch) for one entry point: launch(outs, stream) enqueues it."""
    B, T, H, _ = k.shape
    dev = k.device
    if name in ("fused64", "fused128"):
        C = 64 if name == "fused64" else 128
        outs = [torch.empty((B, T, H, C), dtype=torch.bfloat16, device=dev)]

        def launch(o, s):
            kkt.kkt_solve(k, g, b, cu, chunk_size=C, output_dtype=torch.bfloat16, out=o[0], stream=s)
    elif name in ("gate_cumsum", "gate_cumsum128"):
        C = 64 if name == "gate_cumsum" else 128
        decay = g.clone()
        outs = [torch.empty((B, T, H, C), dtype=torch.float32, device=dev),
                torch.empty((B, T, H), dtype=torch.float32, device=dev)]

        def launch(o, s):
            kkt.kkt_solve_gate_cumsum(k, decay, b, cu, chunk_size=C, output_dtype=torch.float32, out=o[0],
                                      g_out=o[1], stream=s)
    else:  # the two-step chain
        outs = [torch.empty((B, T, H, 64), dtype=torch.float32, device=dev),
                torch.empty((B, T, H, 64), dtype=torch.float16, device=dev)]

        def launch(o, s):
            kkt.kkt_scaled_dot(k, g, b, cu, out=o[0], stream=s)
            kkt.kkt_solve_tril(o[0], cu, output_dtype=torch.float16, out=o[1], stream=s)
    return outs, launch


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("name", ["fused64", "fused128", "gate_cumsum", "gate_cumsum128", "chain"])
def test_graph_replays_equal_eager(kkt, name, packed):
    if packed:
        inp = W.generate("T256_H8_bf16_f32", lengths=[300, 1, 0, 129, 64, 77] + [5, 40] * 40, H=5, seed=7100)
    else:
        inp = W.generate("T256_H8_bf16_f32", B=2, T=1500, H=6, seed=7000)
    say(f"[case] graph capture {name} packed={packed}: T={inp.workload.T} H={inp.workload.H}")
    k, g, b, cu = to_device(inp)
    outs, launch = _calls(kkt, name, k, g, b, cu)
    eager = [torch.empty_like(o) for o in outs]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        launch(eager, s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        launch(outs, s)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            bits = torch.int32 if o.dtype == torch.float32 else torch.int16
            if cu is not None:  # rows outside every sequence stay unwritten in both
                o, e = o[:, : int(cu[-1])], e[:, : int(cu[-1])]
            assert torch.equal(o.view(bits), e.view(bits)), (name, rep)
        if rep == 1:  # new values in the captured input buffers
            k.mul_(-0.5)
            with torch.cuda.stream(s):
                launch(eager, s)
            torch.cuda.synchronize()
