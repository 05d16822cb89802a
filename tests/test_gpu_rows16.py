"""GPU parity of the compact expert rows (moe_experts_rows16, moe_finalize_rows16).

The compact rows come from the same accumulators as moe_experts' fp32 rows,
so the fp32 rows are the exact values they encode: every decoded value must
lie within 2^-11 of its block's largest magnitude (half an fp16 step once the
block maximum is scaled into [2^14, 2^15)), every nonzero block maximum must
scale into that range (or round up to 2^15), and the compact finalize must equal the oracle's
finalize of the decoded rows. The layer end to end (moe_forward, which uses
these calls on the tiled path) is checked against the oracle in the small
and Beam-sized parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_gemm_amd as moe
import synth
from tests.gpu_harness import DEV, Layer, bits, check_layer, log

pytestmark = pytest.mark.gpu

MC = synth.MoEConfig
CASES = [
    MC("r16_ragged", 131, T=150, H=192, E=4, k=2, I=192),       # partial N tiles, 3 blocks per row
    MC("r16_zipf", 132, T=512, H=256, E=16, k=4, I=128, zipf_s=1.1),
    MC("r16_wide", 133, T=700, H=1088, E=8, k=3, I=256),        # a 128 x 512 tail tile per expert
    MC("r16_fp4", 135, T=300, H=512, E=16, k=4, I=256, w_dtype="fp4"),   # quantised tiles
    MC("r16_fp8", 136, T=300, H=576, E=16, k=4, I=192, w_dtype="fp8"),   # 9 blocks per row
    MC("r16_fp4_f8", 137, T=300, H=512, E=16, k=4, I=256, w_dtype="fp4", qmode="f8"),
    MC("r16_fp8_f8_small", 138, T=24, H=256, E=16, k=2, I=128, w_dtype="fp8", qmode="f8"),
]


def run_both(L):
    """The layer's routing and permute, then the experts both ways."""
    c = L.cfg
    r = L.stages()  # compact rows (supported at these sizes)
    assert "y16" in r, "compact rows unsupported at a tiled size"
    ws = moe.workspace(moe.moe_experts_workspace_size(c.T, c.H, c.I, c.E, c.k, L.dw))
    y32 = torch.empty((c.T * c.k, c.H), dtype=torch.float32, device=DEV)
    moe.moe_experts(L.dx, c.I, c.E, c.k, r["offsets"], r["sorted_pair"], L.dw, y32, ws)
    torch.cuda.synchronize()
    return r, y32


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_rows16_encode_fp32_rows(cfg):
    L = Layer(cfg)
    r, y32 = run_both(L)
    P, H = cfg.T * cfg.k, cfg.H
    y = y32.cpu().numpy().astype(np.float64)
    dec = r["y"].cpu().numpy().astype(np.float64)
    v16 = r["y16"].view(torch.float16).float().cpu().numpy().astype(np.float64)
    blk_max = np.abs(y).reshape(P, H // 64, 64).max(axis=2)
    err = np.abs(dec - y).reshape(P, H // 64, 64).max(axis=2)
    assert np.all(err <= blk_max * 2.0 ** -11), f"max err / block max {np.max(err / np.maximum(blk_max, 1e-30)):.3e}"
    scaled_max = np.abs(v16).reshape(P, H // 64, 64).max(axis=2)
    nz = blk_max > 0
    # scaled into [2^14, 2^15) before rounding; the top 8 of the 16384 fp16 steps
    # below 2^15 round up to 2^15 itself
    lo, hi = float(np.min(scaled_max[nz])), float(np.max(scaled_max[nz]))
    n_top = int(np.sum(scaled_max[nz] == 2.0 ** 15))
    assert lo >= 2.0 ** 14 and hi <= 2.0 ** 15, (lo, hi)
    assert np.all(scaled_max[~nz] == 0)
    log(f"[rows16] {cfg.name}: scaled block maxima in [{lo:.1f}, {hi:.1f}], {n_top} rounded up to 2^15 "
        f"of {int(nz.sum())} blocks")
    # finalize over the compact rows = the oracle's finalize of the decoded rows
    ref = oracle.finalize(r["y"].cpu().numpy(), r["pair_pos"].cpu().numpy(), r["w"].cpu().numpy(), cfg.k)
    got = r["out_f32"].cpu().numpy()
    rel = np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2))
    assert rel <= 1e-5, rel
    want = torch.from_numpy(got).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits(r["out"]), want)
    # the layer, and moe_forward bit-identical to the staged compact path
    lay = check_layer(L, r, np.arange(cfg.T))
    f = L.forward()
    assert torch.equal(f["out_f32"], r["out_f32"])
    out = (f"out {lay['out_rel_err']:.2e}" if "decision_matched_rel_err" not in lay else
           f"out decision-matched {lay['decision_matched_rel_err']:.2e} over {lay['checked']} tokens, "
           f"{lay['f8_ambiguous']} F8-ambiguous")
    log(f"[rows16] {cfg.name}: max err/block max {np.max(err / np.maximum(blk_max, 1e-30)):.2e}, "
        f"finalize {rel:.1e}, {out}")


def test_rows16_unsupported_for_streaming_sizes():
    cfg = MC("r16_small", 134, T=16, H=128, E=16, k=2, I=64)  # 2 rows per expert
    L = Layer(cfg)
    r = L.stages()
    assert "y16" not in r
    with pytest.raises(moe.MoEError):
        P = cfg.T * cfg.k
        moe.moe_experts_rows16(L.dx, cfg.I, cfg.E, cfg.k, r["offsets"], r["sorted_pair"], L.dw,
                               torch.empty((P, cfg.H), dtype=torch.int16, device=DEV),
                               torch.empty((P, cfg.H // 64), dtype=torch.uint8, device=DEV),
                               r["experts_ws"])
