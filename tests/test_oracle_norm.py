"""Pins of the oracle's fused finalize + sandwich norm (CPU only).

Each property comes from what an RMS norm is, not from the oracle's formula:
scale invariance, unit RMS of the normalised row, the constant-row case, the
linear regime when eps dominates, per-column gammas, and the bf16 rounding of
the residual (nearest representable value) and of the output.
"""
import numpy as np

import oracle
import synth


def _case(seed, T=5, H=64, k=3, scale=1.0):
    rng = np.random.default_rng(seed)
    P = T * k
    y = (rng.standard_normal((P, H)) * scale).astype(np.float32)
    pair_pos = rng.permutation(P).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    res = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gp = synth.f32_to_bf16_bits((0.5 + rng.random(H)).astype(np.float32))
    gn = synth.f32_to_bf16_bits((0.5 + rng.random(H)).astype(np.float32))
    return y, pair_pos, w, k, res, gp, gn


def test_post_norm_is_scale_invariant_and_unit_rms():
    y, pp, w, k, res, gp, gn = _case(1)
    ones = synth.f32_to_bf16_bits(np.ones(y.shape[1], np.float32))
    a = oracle.finalize_norm(y, pp, w, k, res, ones, gn, 0.0)
    b = oracle.finalize_norm(y * np.float32(8.0), pp, w, k, res, ones, gn, 0.0)  # exact scaling
    np.testing.assert_allclose(b["post"], a["post"], rtol=1e-13, atol=0)
    np.testing.assert_allclose(np.mean(a["post"] ** 2, axis=1), 1.0, rtol=1e-13)
    # the same with gammas: post / gamma has unit RMS
    c = oracle.finalize_norm(y, pp, w, k, res, gp, gn, 0.0)
    g = oracle.format_op("bf16", gp)
    np.testing.assert_allclose(np.mean((c["post"] / g) ** 2, axis=1), 1.0, rtol=1e-13)


def test_constant_rows_and_eps_regimes():
    T, H, k = 4, 64, 2
    rng = np.random.default_rng(2)
    v = rng.standard_normal(H).astype(np.float32)
    y = np.tile(v, (T * k, 1))
    pp = np.arange(T * k, dtype=np.int32)
    w = np.full((T, k), 0.5, np.float32)       # weights sum to 1: m = v exactly
    res = np.zeros((T, H), np.uint16)
    gp = synth.f32_to_bf16_bits(np.full(H, 2.0, np.float32))
    gn = synth.f32_to_bf16_bits(np.ones(H, np.float32))
    out = oracle.finalize_norm(y, pp, w, k, res, gp, gn, 0.0)
    vd = v.astype(np.float64)
    np.testing.assert_allclose(out["m"], np.tile(vd, (T, 1)), rtol=0, atol=0)
    np.testing.assert_allclose(out["post"], np.tile(2.0 * vd / np.sqrt(np.mean(vd * vd)), (T, 1)),
                               rtol=1e-14)
    # eps far above mean(m^2): the norm becomes a fixed scale 1/sqrt(eps)
    big = oracle.finalize_norm(y, pp, w, k, res, gp, gn, 1e12)
    np.testing.assert_allclose(big["post"], np.tile(2.0 * vd / 1e6, (T, 1)), rtol=1e-9)


def test_gamma_is_per_column():
    y, pp, w, k, res, gp, gn = _case(3)
    H = y.shape[1]
    perm = np.random.default_rng(4).permutation(H)
    a = oracle.finalize_norm(y, pp, w, k, res, gp, gn, 1e-6)
    b = oracle.finalize_norm(y[:, perm], pp, w, k, res[:, perm], gp[perm], gn[perm], 1e-6)
    # (the row mean sums in another order: equal to fp64 rounding)
    np.testing.assert_allclose(b["post"], a["post"][:, perm], rtol=1e-13, atol=0)
    for key in ("r", "normed"):
        np.testing.assert_array_equal(b[key], a[key][:, perm])


def test_residual_and_output_rounding():
    y, pp, w, k, res, gp, gn = _case(5, T=7, H=128)
    out = oracle.finalize_norm(y, pp, w, k, res, gp, gn, 1e-6)
    exact = oracle.format_op("bf16", res) + out["post"]
    r = out["r"]
    # r is bf16-representable and the nearest such value to the exact sum
    assert np.array_equal(oracle.format_op("round_bf16", r), r)
    ulp = np.abs(np.nextafter(r.astype(np.float32), np.float32(np.inf)) - r.astype(np.float32))
    ulp = np.where(np.abs(r) > 0, np.ldexp(1.0, np.frexp(np.abs(r))[1] - 8), ulp)
    assert np.all(np.abs(r - exact) <= ulp / 2 + 1e-300)
    # the next norm reads the rounded residual
    nn = oracle.rms_norm(r, oracle.format_op("bf16", gn), 1e-6)
    assert np.array_equal(out["normed"], oracle.format_op("round_bf16", nn))
    # rows are independent: a subset of tokens gives the same rows
    sub = oracle.finalize_norm(y, pp, w, k, res, gp, gn, 1e-6, rows=np.array([2, 5]))
    assert np.array_equal(sub["normed"], out["normed"][[2, 5]])
