"""CPU checks of the GPU harness's own logic (no GPU needed).

The fp8-MFMA-mode parity check classifies every E4M3 code of h that differs
between the kernel's h and the oracle's as a rounding-boundary decision or a
failure, and composes the oracle's F8 layer from its steps to get at h. Both
are checked here against the oracle itself and against planted cases: a real
boundary decision must be accepted and counted, a code that no rounding
boundary explains must fail.
"""
import types

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_harness import (bf16_ulp, check_h_rows, e4m3_spacing, f8_decisions, f8_h_codes,
                               layer_ref_f8)


def _layer(cfg):
    wr, bias = synth.gen_router(cfg)
    return types.SimpleNamespace(cfg=cfg, x=synth.gen_x(cfg), wr=wr, bias=bias,
                                 hw=synth.gen_experts(cfg))


@pytest.mark.parametrize("wdt", ["fp4", "fp8"])
def test_composed_f8_layer_equals_oracle_layer(wdt):
    """The harness's F8 reference (logits, routing, expert rows, slot-ordered sum)
    is oracle.layer in the fp8-MFMA mode, bit for bit."""
    cfg = synth.MoEConfig("f8_compose", 41, T=24, H=256, E=8, k=3, I=192, w_dtype=wdt, qmode="f8")
    L = _layer(cfg)
    tok = np.array([0, 3, 5, 11, 23])
    ref = layer_ref_f8(L, tok)
    want = oracle.layer(L.x, L.wr, L.bias, L.hw, cfg.I, cfg.k, "bf16", rows=tok, qmode="f8")
    assert np.array_equal(ref["out"], want["out"])
    assert np.array_equal(ref["ids"], want["ids"])
    assert np.array_equal(ref["w"], want["w"])


def test_h_codes_match_the_oracle_encoding():
    cfg = synth.MoEConfig("f8_codes", 42, T=16, H=256, E=4, k=2, I=320, w_dtype="fp4", qmode="f8")
    L = _layer(cfg)
    tok = np.arange(16).repeat(2)
    ex = np.tile([0, 3], 16)
    _, h, hq = oracle.expert_rows_f8(L.x, L.hw, cfg.I, tok, ex, want_h=True)
    assert np.array_equal(f8_h_codes(h, cfg.I)[0], hq)  # includes a partial 64-column block


def test_spacings():
    assert bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([1.99]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([-3.0]))[0] == 2.0 ** -6
    assert e4m3_spacing(np.array([1.0]))[0] == 0.125
    assert e4m3_spacing(np.array([448.0]))[0] == 32.0
    assert e4m3_spacing(np.array([0.0]))[0] == 2.0 ** -9
    assert e4m3_spacing(np.array([2.0 ** -6]))[0] == 2.0 ** -9
    grid = np.unique(np.abs(oracle.format_op("e4m3", np.arange(127))))
    for a, b in zip(grid[:-1], grid[1:]):  # the spacing is the gap to the next grid value
        assert b - a == e4m3_spacing(np.array([a]))[0]


def _row(values, I=128):
    h = np.zeros((1, I))
    h[0, :len(values)] = values
    h[0, -1] = 400.0  # block max: exponent 0 (448 >= 400 > 224)
    return h


def test_boundary_decision_is_accepted_and_counted():
    # 1.0625 is the E4M3 midpoint between 1.0 and 1.125 (exponent 0); bf16
    # neighbours on each side of it round to different codes
    lo, hi = 1.0625 - 2.0 ** -7, 1.0625
    hr, hg = _row([lo]), _row([hi])
    assert f8_h_codes(hr, 128)[0][0, 0] == 1.0 and f8_h_codes(hg, 128)[0][0, 0] == 1.0  # tie to even
    hg = _row([1.0625 + 2.0 ** -7])
    assert f8_h_codes(hg, 128)[0][0, 0] == 1.125
    touched, n_code, n_blk = f8_decisions(hg, hr, 128, "planted")
    assert touched[0] and n_code == 1 and n_blk == 0


def test_same_values_same_codes():
    h = _row(np.linspace(-3, 3, 100))
    touched, n_code, n_blk = f8_decisions(h, h.copy(), 128, "same")
    assert not touched.any() and n_code == 0 and n_blk == 0


def test_unexplained_code_fails():
    # three E4M3 steps apart, beyond the h tolerance: no rounding boundary explains it
    hr, hg = _row([1.0]), _row([1.375])
    with pytest.raises(AssertionError):
        f8_decisions(hg, hr, 128, "planted")
    with pytest.raises(AssertionError):
        check_h_rows(hg, hr, "planted")


def test_block_exponent_straddle_is_a_boundary():
    # block maxima 224 - step and 224 + step straddle 448 * 2^-1
    hr = np.zeros((1, 128))
    hg = np.zeros((1, 128))
    hr[0, 0], hg[0, 0] = 224.0, 225.0
    assert f8_h_codes(hr, 128)[1][0, 0] == -1 and f8_h_codes(hg, 128)[1][0, 0] == 0
    touched, _, n_blk = f8_decisions(hg, hr, 128, "planted")
    assert touched[0] and n_blk == 1
    hg[0, 0] = 900.0  # two exponents apart
    with pytest.raises(AssertionError):
        f8_decisions(hg, hr, 128, "planted")


def test_tiny_values_may_cross_several_steps_in_order():
    # a near-cancelled h within the fp32 floor (2^-12 of the row max) may move
    # over several grid steps, even across zero, as long as the codes follow the
    # values
    hr, hg = _row([-0.003]), _row([0.004])
    touched, n_code, _ = f8_decisions(hg, hr, 128, "tiny")
    assert touched[0] and n_code == 1
    check_h_rows(hg, hr, "tiny")  # 0.007 <= 400 * 2^-12


def test_h_rows_within_one_bf16_step():
    hr = np.linspace(0.5, 3.0, 64)[None, :]
    hg = hr + bf16_ulp(hr)
    check_h_rows(hg, hr, "one step")
    hg[0, 5] += bf16_ulp(hr[:, 5:6])[0, 0] * 2
    with pytest.raises(AssertionError):
        check_h_rows(hg, hr, "three steps")
