"""moe_forward_noalloc (the whole layer on the library's own scratch area, for
callers that cannot allocate) against moe_forward with a caller workspace.

Both run the same kernels, so every output must agree bit for bit. Consecutive
calls share the scratch area and leave their contents in it; each call here is
smaller than the one before (tiled grouped GEMMs with compact rows, then the
streaming kernels, the fp8-MFMA mode, split K with h formed in the down
kernel, and one token), so a call that read stale bytes of a larger earlier
call would show up as a mismatch.
"""
import numpy as np
import pytest
import torch

import sparse_moe_layer_gemm_amd as moe
import synth

pytestmark = pytest.mark.gpu

MC = synth.MoEConfig
H, E, k = 1024, 64, 8
SEQ = [
    MC("noalloc_tiled", 301, T=320, H=H, E=E, k=k, I=512),            # 2560 pairs: tiled, compact rows
    MC("noalloc_stream", 301, T=96, H=H, E=E, k=k, I=512),            # streaming kernels
    MC("noalloc_f8_fp4", 302, T=64, H=H, E=E, k=k, I=512, w_dtype="fp4", qmode="f8"),
    MC("noalloc_fold", 301, T=3, H=H, E=E, k=k, I=512),               # split K, h formed in LDS
    MC("noalloc_one_token", 301, T=1, H=H, E=E, k=k, I=512),          # permute inside the select
]


def _inputs(cfg, cache={}):
    key = (cfg.seed, cfg.w_dtype)
    if key not in cache:
        cache[key] = moe.experts_to_device(synth.gen_experts(cfg.with_(T=1)))
    dw = cache[key]
    if cfg.qmode == "f8":
        import dataclasses
        dw = dataclasses.replace(dw, qmode=moe.MOE_QMODE_F8)
    x = moe.to_device_bf16(synth.gen_x(cfg))
    wr, bias = synth.gen_router(cfg)
    return x, torch.from_numpy(wr).cuda(), dw


def _outputs(cfg):
    T = cfg.T
    return {"out": torch.empty((T, H), dtype=torch.bfloat16, device="cuda"),
            "out_f32": torch.empty((T, H), dtype=torch.float32, device="cuda"),
            "logits": torch.empty((T, E), dtype=torch.bfloat16, device="cuda"),
            "ids": torch.empty((T, k), dtype=torch.int32, device="cuda"),
            "w": torch.empty((T, k), dtype=torch.float32, device="cuda")}


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _run_pair(cfg, stream=None):
    x, wr, dw = _inputs(cfg)
    ref = _outputs(cfg)
    ws = moe.workspace(moe.moe_forward_workspace_size(cfg.T, H, cfg.I, E, k, dw))
    assert ws.numel() <= moe.NOALLOC_SCRATCH_BYTES
    moe.moe_forward(x, wr, None, dw, cfg.I, k, ref["out"], ws, out_f32=ref["out_f32"],
                    logits=ref["logits"], topk_ids=ref["ids"], topk_w=ref["w"], stream=stream)
    got = _outputs(cfg)
    moe.moe_forward_noalloc(x, wr, None, dw, cfg.I, k, got["out"], out_f32=got["out_f32"],
                            logits=got["logits"], topk_ids=got["ids"], topk_w=got["w"],
                            stream=stream)
    torch.cuda.synchronize()
    for name in ref:
        assert _same(ref[name], got[name]), f"{cfg.name}: {name} differs from moe_forward"
    return ref


def test_noalloc_matches_forward_on_shrinking_calls():
    for cfg in SEQ:
        print(f"[noalloc] {cfg.name} T={cfg.T} w={cfg.w_dtype} qmode={cfg.qmode}", flush=True)
        ref = _run_pair(cfg)
        assert torch.isfinite(ref["out_f32"]).all()


def test_noalloc_twice_in_a_row_smaller_second():
    """Two calls in a row on the scratch area, the second with a smaller input,
    each against moe_forward; the first call's outputs are unchanged by the second."""
    a, b = SEQ[0], SEQ[1].with_(name="noalloc_second", seed=303)
    first = _run_pair(a)
    keep = {n: t.clone() for n, t in first.items()}
    _run_pair(b)
    for n in keep:
        assert _same(keep[n], first[n])


def test_noalloc_on_a_side_stream():
    """The device comes from the stream; work is ordered on that stream."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        _run_pair(SEQ[1].with_(name="noalloc_side_stream"), stream=s)


def test_noalloc_rejects_sizes_beyond_the_scratch_area():
    cfg = MC("noalloc_too_big", 304, T=16384, H=H, E=E, k=k, I=512)
    x = torch.empty((cfg.T, H), dtype=torch.bfloat16, device="cuda")
    wr = torch.empty((H, E), dtype=torch.float32, device="cuda")
    _, _, dw = _inputs(SEQ[1])
    assert moe.moe_forward_workspace_size(cfg.T, H, cfg.I, E, k, dw) > moe.NOALLOC_SCRATCH_BYTES
    out = torch.empty((cfg.T, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as err:
        moe.moe_forward_noalloc(x, wr, None, dw, cfg.I, k, out)
    assert err.value.status == 3  # MOE_ERR_WORKSPACE_TOO_SMALL, nothing enqueued
