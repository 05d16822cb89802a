"""GPU parity of the fused finalize + sandwich norms (moe_finalize_norm) against
the oracle's finalize_norm (MI355X).

The residual is checked against the oracle's exact pre-rounding value v =
residual + post: the kernel's bf16 residual must lie between RNE(v - d) and
RNE(v + d), d = 1e-5 x the row's max |v| (the sum can cancel, so fp32 error is
absolute at the row's scale; only values within d of a bf16 rounding midpoint
may round the other way, and their count is reported). The next sublayer's
input is checked stage by stage from the oracle's norm u of the kernel's own
residual, with d = 1e-5 |u| per element (a product: relative error). In-place update, determinism and degenerate
shapes are covered too.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_gemm_amd as moe
import synth
from tests.gpu_harness import DEV, Layer, bits, log

pytestmark = pytest.mark.gpu

REL = 1e-5


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


def to_bf16(bits_u16):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def bracket(got, exact, d):
    """got (bf16 values) lies between RNE(v - d) and RNE(v + d); returns the count
    of elements that differ from RNE(v)."""
    lo = oracle.format_op("round_bf16", exact - d)
    hi = oracle.format_op("round_bf16", exact + d)
    bad = (got < lo) | (got > hi)
    assert not bad.any(), f"{int(bad.sum())} values outside the rounding bracket"
    return int(np.sum(got != oracle.format_op("round_bf16", exact)))


def run(y, pp, w, res, gp, gn, eps, in_place=False):
    dy = torch.from_numpy(y).to(DEV)
    dpp = torch.from_numpy(pp).to(DEV)
    dw = torch.from_numpy(w).to(DEV)
    dres, dgp, dgn = to_bf16(res), to_bf16(gp), to_bf16(gn)
    normed = torch.empty_like(dres)
    out = dres if in_place else torch.empty_like(dres)
    moe.moe_finalize_norm(dy, dpp, dw, dres, dgp, dgn, eps, out, normed)
    torch.cuda.synchronize()
    return bits(out), bits(normed)


def check(y, pp, w, res, gp, gn, eps, k):
    r_bits, n_bits = run(y, pp, w, res, gp, gn, eps)
    ref = oracle.finalize_norm(y, pp, w, k, res, gp, gn, eps)
    v = oracle.format_op("bf16", res) + ref["post"]
    r = oracle.format_op("bf16", r_bits)
    # residual + post can cancel: fp32 error is absolute, at the row's scale
    flips_r = bracket(r, v, REL * np.max(np.abs(v), axis=1, keepdims=True))
    # next norm, from the kernel's own residual: a product, so relative error
    gnv = oracle.format_op("bf16", gn)
    u = oracle.rms_norm(r, gnv, eps)
    n = oracle.format_op("bf16", n_bits)
    flips_n = bracket(n, u, REL * np.abs(u))
    # end to end against the oracle's rounded outputs: the residual within one
    # bf16 step plus the row-scale bracket; the normed value moves with the
    # residual's difference times the row's scale factor, plus one bf16 step
    step = 2.0 ** -7
    dr = np.abs(r - ref["r"])
    assert np.all(dr <= np.abs(ref["r"]) * step + 2 * REL * np.max(np.abs(v), axis=1, keepdims=True))
    scale = gnv / np.sqrt(np.mean(ref["r"] ** 2, axis=1, keepdims=True) + eps)
    dn = np.abs(n - ref["normed"])
    assert np.all(dn <= dr * scale * (1 + 2 * step) + np.abs(ref["normed"]) * step)
    log(f"finalize_norm T={w.shape[0]} H={y.shape[1]} k={k}: residual {flips_r}, normed {flips_n} "
        f"values round the other way; {int(np.sum(dr > 0))} residual values differ from the "
        f"oracle's")
    return r_bits, n_bits


@pytest.mark.parametrize("T,H,k,eps", [
    (128, 5120, 8, 1e-6),    # Beam decode shape: 2 column chunks per lane, the second partial
    (37, 192, 3, 1e-5),      # ragged: 48 of 1024 lanes hold a chunk
    (16, 1088, 1, 1e-6),     # 272 of 1024 lanes; k = 1
    (5, 16384, 8, 1e-6),     # widest row: 4 full chunks per lane
    (1, 64, 2, 0.0),         # smallest row (16 lanes), no epsilon
])
def test_finalize_norm_parity(T, H, k, eps):
    y, pp, w, res, gp, gn = make_inputs(11, T, H, k)
    check(y, pp, w, res, gp, gn, eps, k)


def test_finalize_norm_eps_dominated_rows():
    # tiny expert rows: eps dominates mean(m^2), post ~ m / sqrt(eps)
    y, pp, w, res, gp, gn = make_inputs(12, 24, 256, 4, y_scale=1e-5)
    check(y, pp, w, res, gp, gn, 1e-6, 4)


def test_finalize_norm_in_place_and_deterministic():
    y, pp, w, res, gp, gn = make_inputs(13, 300, 5120, 8)
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
