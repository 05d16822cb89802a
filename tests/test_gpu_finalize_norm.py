"""GPU parity of the fused finalize + sandwich norms (moe_finalize_norm, its
compact-row form and the layer ending in it, moe_forward_norm) against the
oracle's finalize_norm (MI355X).

The residual is checked against the oracle's exact pre-rounding value v =
residual + post: the kernel's bf16 residual must lie between RNE(v - d) and
RNE(v + d), d = 1e-5 x the row's max |v| (the sum can cancel, so fp32 error is
absolute at the row's scale), and equal the oracle's rounded residual wherever
those two agree; values at a rounding boundary are counted. The next
sublayer's input is checked stage by stage from the oracle's norm u of the
kernel's own residual, with d = 1e-5 |u| per element (a product: relative
error). In-place update, determinism and degenerate shapes are covered too.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_gemm_amd as moe
import synth
from tests.gpu_harness import (DEV, Layer, bits, check_norm_outputs, forward_norm_vs_stages, log,
                               to_bf16_dev)

pytestmark = pytest.mark.gpu

def make_inputs(seed, T, H, k, y_scale=1.0):
    """Seeded synthetic inputs: fp32 expert rows, a permutation of the pair
    positions, renormalised weights, a bf16 residual and bf16 norm weights."""
    rng = np.random.default_rng([seed, T, H, k])
    P = T * k
    y = (rng.standard_normal((P, H)) * y_scale).astype(np.float32)
    pp = rng.permutation(P).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32) + np.float32(0.05)
    w /= w.sum(1, keepdims=True)
    res = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gp = synth.f32_to_bf16_bits((0.5 + rng.random(H)).astype(np.float32))
    gn = synth.f32_to_bf16_bits((0.5 + rng.random(H)).astype(np.float32))
    return y, pp, w, res, gp, gn


def run(y, pp, w, res, gp, gn, eps, in_place=False):
    dy = torch.from_numpy(y).to(DEV)
    dpp = torch.from_numpy(pp).to(DEV)
    dw = torch.from_numpy(w).to(DEV)
    dres, dgp, dgn = to_bf16_dev(res), to_bf16_dev(gp), to_bf16_dev(gn)
    normed = torch.empty_like(dres)
    out = dres if in_place else torch.empty_like(dres)
    moe.moe_finalize_norm(dy, dpp, dw, dres, dgp, dgn, eps, out, normed)
    torch.cuda.synchronize()
    return bits(out), bits(normed)


def check(y, pp, w, res, gp, gn, eps, k):
    r_bits, n_bits = run(y, pp, w, res, gp, gn, eps)
    check_norm_outputs(y, pp, w, k, res, gp, gn, eps, r_bits, n_bits)
    return r_bits, n_bits


@pytest.mark.parametrize("T,H,k,eps", [
    (128, 5120, 8, 1e-6),    # Beam decode shape: 2 column chunks per lane, the second partial
    (37, 192, 3, 1e-5),      # ragged: 48 of 1024 lanes hold a chunk
    (16, 1088, 1, 1e-6),     # 272 of 1024 lanes; k = 1
    (5, 16384, 8, 1e-6),     # widest row: 4 full chunks per lane
    (1, 64, 2, 0.0),         # smallest row (16 lanes), no epsilon
    # from 1024 tokens on, 256 lanes per token
    (1100, 5120, 8, 1e-6),   # 5 chunks per lane
    (1024, 1088, 3, 1e-5),   # 2 chunks, the second on 16 of 256 lanes
    (1030, 6144, 8, 1e-6),   # 6 chunks per lane, the most the 256-lane form takes
    (1040, 8192, 4, 1e-6),   # wider rows: back to 1024 lanes per token
])
def test_finalize_norm_parity(T, H, k, eps):
    y, pp, w, res, gp, gn = make_inputs(11, T, H, k)
    check(y, pp, w, res, gp, gn, eps, k)


def test_finalize_norm_eps_dominated_rows():
    # tiny expert rows: eps dominates mean(m^2), post ~ m / sqrt(eps)
    y, pp, w, res, gp, gn = make_inputs(12, 24, 256, 4, y_scale=1e-5)
    check(y, pp, w, res, gp, gn, 1e-6, 4)


@pytest.mark.parametrize("T", [300, 1500])
def test_finalize_norm_in_place_and_deterministic(T):
    y, pp, w, res, gp, gn = make_inputs(13, T, 5120, 8)
    a = run(y, pp, w, res, gp, gn, 1e-6)
    b = run(y, pp, w, res, gp, gn, 1e-6, in_place=True)
    c = run(y, pp, w, res, gp, gn, 1e-6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_finalize_norm_empty_batch():
    H = 128
    dy = torch.empty((0, H), dtype=torch.float32, device=DEV)
    dpp = torch.empty((0,), dtype=torch.int32, device=DEV)
    dw = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    dres = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    moe.moe_finalize_norm(dy, dpp, dw, dres, g, g, 1e-6, dres, torch.empty_like(dres))
    torch.cuda.synchronize()


def test_finalize_norm_after_the_layer():
    # on the expert rows, positions and weights the layer's own stages produce
    cfg = synth.MoEConfig("fn_layer", 121, T=96, H=512, E=16, k=4, I=128)
    L = Layer(cfg)
    r = L.stages()
    y = r["y"].cpu().numpy()
    pp = r["pair_pos"].cpu().numpy()
    w = r["w"].cpu().numpy()
    rng = np.random.default_rng(121)
    res = synth.f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.H)).astype(np.float32))
    gp = synth.f32_to_bf16_bits((0.5 + rng.random(cfg.H)).astype(np.float32))
    gn = synth.f32_to_bf16_bits((0.5 + rng.random(cfg.H)).astype(np.float32))
    check(y, pp, w, res, gp, gn, 1e-6, cfg.k)


# The layer ending in the fused step: compact rows on the tiled kernels, fp32
# rows on the streaming ones, and a split-K down GEMM (whose partial sums are
# reduced before the fused step), each bit for bit against the stages and
# against the oracle on the layer's own rows.
@pytest.mark.parametrize("cfg", [
    synth.MoEConfig("fwdnorm_tiled", 131, T=300, H=512, E=16, k=4, I=256),
    synth.MoEConfig("fwdnorm_stream", 132, T=40, H=640, E=32, k=4, I=128),
    synth.MoEConfig("fwdnorm_split", 133, T=2, H=1024, E=64, k=3, I=320),
    synth.MoEConfig("fwdnorm_fp4_f8", 134, T=200, H=256, E=8, k=4, I=192, w_dtype="fp4",
                    qmode="f8"),
    synth.MoEConfig("fwdnorm_one_token", 135, T=1, H=256, E=8, k=8, I=128),
], ids=lambda c: c.name)
def test_forward_norm_paths(cfg):
    L = Layer(cfg)
    r = L.stages()
    forward_norm_vs_stages(L, r)


def test_finalize_norm_rows16_matches_fp32_rows():
    """The compact-row fused step decodes each value exactly: the same outputs as
    the fp32-row step on the decoded rows."""
    cfg = synth.MoEConfig("fn_rows16", 136, T=256, H=384, E=8, k=4, I=128)
    L = Layer(cfg)
    r = L.stages()
    assert "y16" in r
    res, gp, gn = (to_bf16_dev(a) for a in make_inputs(136, cfg.T, cfg.H, cfg.k)[3:])
    a_r, a_n, b_r, b_n = (torch.empty_like(res) for _ in range(4))
    moe.moe_finalize_norm_rows16(r["y16"], r["y16_scale"], r["pair_pos"], r["w"], res, gp, gn, 1e-6,
                                 a_r, a_n)
    moe.moe_finalize_norm(r["y"], r["pair_pos"], r["w"], res, gp, gn, 1e-6, b_r, b_n)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a_r), bits(b_r)) and np.array_equal(bits(a_n), bits(b_n))
