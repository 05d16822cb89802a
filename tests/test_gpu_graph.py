"""moe_forward captured in a HIP graph (MI355X).

The library allocates nothing, syncs nothing and clears no memory with
hipMemsetAsync, so a whole layer can be captured once and replayed. Each case
captures `moe_forward` on static buffers, then replays the graph several times
with the program's own eager work and synchronisations in between (the output
is overwritten eagerly before each replay, and the input changes once), and
checks every replay bit for bit against an eager call on the same input.
The cases cover the three expert paths: streaming with split K (few rows per
expert), streaming without it, and the tiled kernels (many rows per expert),
for bf16 and NVFP4 weights; a single token (its select kernel also writes the
permutation); and the fp8-MFMA mode (its quantiser kernels in the graph too).
"""
import pytest
import torch

import sparse_moe_layer_gemm_amd as moe
import synth
from tests.gpu_harness import Layer, log

pytestmark = pytest.mark.gpu

MC = synth.MoEConfig
CASES = [
    MC("graph_split_k", 201, T=2, H=512, E=32, k=4, I=256),
    MC("graph_stream", 202, T=40, H=256, E=16, k=2, I=128),
    MC("graph_tiled", 203, T=512, H=256, E=16, k=4, I=128, zipf_s=1.1),
    MC("graph_fp4_tiled", 204, T=300, H=512, E=16, k=4, I=256, w_dtype="fp4"),
    MC("graph_one_token", 205, T=1, H=512, E=32, k=4, I=256),
    MC("graph_fp4_stream", 206, T=8, H=512, E=16, k=2, I=256, w_dtype="fp4"),
    MC("graph_f8_tiled", 207, T=300, H=256, E=8, k=4, I=192, w_dtype="fp4", qmode="f8"),
]


def _outputs(cfg, dx):
    T, H, k = cfg.T, cfg.H, cfg.k
    return {"out": torch.empty((T, H), dtype=dx.dtype, device="cuda"),
            "out_f32": torch.empty((T, H), dtype=torch.float32, device="cuda"),
            "ids": torch.empty((T, k), dtype=torch.int32, device="cuda"),
            "w": torch.empty((T, k), dtype=torch.float32, device="cuda")}


def _call(L, x, o, ws):
    c = L.cfg
    moe.moe_forward(x, L.dwr, L.dbias, L.dw, c.I, c.k, o["out"], ws, out_f32=o["out_f32"],
                    topk_ids=o["ids"], topk_w=o["w"])


def _same(a: dict, b: dict) -> bool:
    return all(torch.equal(a[n].view(torch.int16) if a[n].dtype == torch.bfloat16 else a[n],
                           b[n].view(torch.int16) if b[n].dtype == torch.bfloat16 else b[n])
               for n in a)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_graph_replays(cfg):
    log(f"[graph] {cfg.name}")
    L = Layer(cfg)
    c = cfg
    ws = moe.workspace(moe.moe_forward_workspace_size(c.T, c.H, c.I, c.E, c.k, L.dw))
    x = L.dx.clone()                      # the graph's static input
    x2 = (L.dx.float() * -0.75).to(L.dx.dtype)  # a second input, copied in before a replay

    ref = _outputs(cfg, x)
    _call(L, x, ref, ws)
    ref2 = _outputs(cfg, x)
    _call(L, x2, ref2, ws)
    torch.cuda.synchronize()

    o = _outputs(cfg, x)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        _call(L, x, o, ws)                # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(L, x, o, ws)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in o.values():              # eager work between replays
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(o, ref), f"replay {rep} differs from the eager call"
    x.copy_(x2)                           # new input in the captured buffer
    g.replay()
    torch.cuda.synchronize()
    assert _same(o, ref2), "replay on a new input differs from the eager call"
    x.copy_(L.dx)
    g.replay()
    torch.cuda.synchronize()
    assert _same(o, ref)
