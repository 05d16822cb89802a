"""Pins of the oracle's fp8-MFMA ("F8") mode of the quantised experts (CPU only).

The F8 mode encodes every GEMM operand as E4M3: per-token scaled activations,
NVFP4 weights re-encoded to E4M3, h per (row, 128-column block) with a
power-of-two scale. Each piece is pinned against something outside the oracle:
the E4M3 grid of the format decoder (itself pinned to the OCP tables), the
defining properties of round-to-nearest-even and of the smallest covering
power of two, lossless cases that must reproduce the (separately pinned)
exact-dequantisation path, and NumPy matmuls of the oracle's own quantised
operands.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.test_oracle import _exact_quantised_case


def _e4m3_grid():
    v = oracle.format_op("e4m3", np.arange(256))
    v = v[np.isfinite(v)]
    return np.unique(v)


def test_round_e4m3_grid_ties_and_saturation():
    grid = _e4m3_grid()
    assert grid.max() == 448.0 and grid.min() == -448.0
    # every representable value is fixed
    assert np.array_equal(oracle.format_op("round_e4m3", grid), grid)
    pos = grid[grid >= 0]
    codes = {float(v): c for c, v in enumerate(oracle.format_op("e4m3", np.arange(128)))}
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2
    got = oracle.format_op("round_e4m3", mid)
    # ties go to the neighbour whose code is even (last mantissa bit 0)
    want = np.where([codes[float(a)] % 2 == 0 for a in lo], lo, hi)
    assert np.array_equal(got, want)
    # just off the midpoint: the nearer neighbour
    eps = (hi - lo) * 1e-6
    assert np.array_equal(oracle.format_op("round_e4m3", mid - eps), lo)
    assert np.array_equal(oracle.format_op("round_e4m3", mid + eps), hi)
    assert np.array_equal(oracle.format_op("round_e4m3", -(mid + eps)), -hi)
    # saturation at the largest finite value
    assert np.array_equal(oracle.format_op("round_e4m3", [449.0, 500.0, 1e9, -1e9]),
                          [448.0, 448.0, 448.0, -448.0])


def test_block_exp_is_smallest_covering_power_of_two():
    rng = np.random.default_rng(3)
    amax = np.concatenate([2.0 ** rng.uniform(-100, 100, 2000), 448.0 * 2.0 ** np.arange(-20, 21),
                           np.nextafter(448.0 * 2.0 ** np.arange(-20, 21), np.inf), [1.0, 3.5, 1e-30]])
    e = oracle.format_op("block_exp", amax)
    assert np.all(e == np.round(e))
    covers = 448.0 * 2.0 ** e >= amax
    minimal = 448.0 * 2.0 ** (e - 1) < amax
    assert np.all(covers) and np.all(minimal)
    assert oracle.format_op("block_exp", [0.0])[0] == 0.0
    # the E8M0 range clamps
    assert oracle.format_op("block_exp", [2.0 ** -200, 2.0 ** 200]).tolist() == [-127.0, 127.0]


def test_quantize_x_properties():
    rng = np.random.default_rng(4)
    T, H = 12, 256
    xf = rng.standard_normal((T, H)) * 2.0 ** rng.integers(-20, 20, (T, 1))
    xf[3] = 0.0
    x = synth.f32_to_bf16_bits(xf.astype(np.float32))
    xb = synth.bf16_bits_to_f32(x).astype(np.float64)
    xq, s = oracle.quantize_x(x)
    grid = _e4m3_grid()
    assert np.all(np.isin(xq, grid))
    amax = np.abs(xb).max(1)
    for t in range(T):
        if amax[t] == 0:
            assert s[t] == 1.0 and np.all(xq[t] == 0)
            continue
        assert s[t] == np.float32(amax[t]) / np.float32(448.0)  # one fp32 division
        r = (xb[t].astype(np.float32) / s[t]).astype(np.float64)  # the fp32 quotient
        # nearest grid point (the grid's spacing bounds the error)
        idx = np.searchsorted(grid, r)
        below, above = grid[np.clip(idx - 1, 0, grid.size - 1)], grid[np.clip(idx, 0, grid.size - 1)]
        dist = np.minimum(np.abs(r - below), np.abs(r - above))
        assert np.all(np.abs(xq[t] - r) <= dist + 1e-300)
        assert np.abs(xq[t]).max() == 448.0  # the row's largest value lands on the top code


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_f8_gate_up_equals_exact_path_when_lossless(fmt):
    """x on the E4M3 grid with each row's amax = 448 (scale 1) and weights whose
    E4M3 re-encoding is exact: the F8 h equals the exact path's h rounded to bf16."""
    rng = np.random.default_rng(21)
    T, H, I, E = 5, 64, 64, 3
    q, _ = _exact_quantised_case(rng, E, H, I, fmt)
    grid = _e4m3_grid()
    small = grid[(np.abs(grid) <= 4) & (np.abs(grid) >= 2.0 ** -3)]
    xv = small[rng.integers(0, small.size, (T, H))]
    xv[:, 0] = 448.0
    x = synth.f32_to_bf16_bits(xv.astype(np.float32))
    tok = np.repeat(np.arange(T), E)
    eid = np.tile(np.arange(E), T)
    _, h8, _ = oracle.expert_rows_f8(x, q, I, tok, eid, want_h=True)
    _, hw = oracle.expert_rows(x, q, I, tok, eid, want_h=True)
    hw_b = oracle.format_op("round_bf16", hw)
    agree = np.mean(h8 == hw_b)
    assert agree > 0.995, agree
    np.testing.assert_allclose(h8, hw_b, rtol=2.0 ** -7, atol=1e-30)


def _w8_matrices(q, fmt, E, H, I):
    """The E4M3 operand values of the F8 mode, built from the format tables:
    gate/up [E, H, 2I] and down [E, I, H] (K-major rows), and the column scales."""
    e4 = oracle.format_op("e4m3", np.arange(256))
    e2 = oracle.format_op("e2m1", np.arange(16))

    def mat(codes, scales, gsc, N, K):
        if fmt == "fp8":
            return e4[codes.reshape(E, N, K)], scales.astype(np.float64)
        lo, hi = codes & 15, codes >> 4
        nib = np.stack([lo, hi], -1).reshape(E, N, K)
        blk = np.repeat(e4[scales.reshape(E, N, K // 16)], 16, axis=2)
        v = oracle.format_op("round_e4m3", e2[nib] * blk / 8.0)
        return v, 8.0 * np.repeat(gsc.astype(np.float64)[:, None], N, axis=1)

    gu, sgu = mat(q["gate_up"], q["gate_up_scale"], q.get("gate_up_gscale"), 2 * I, H)
    dn, sdn = mat(q["down"], q["down_scale"], q.get("down_gscale"), H, I)
    return gu, sgu, dn, sdn


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_f8_rows_match_numpy_on_quantised_operands(fmt):
    rng = np.random.default_rng(22)
    T, H, I, E = 6, 64, 192, 3  # I = 192: one full and one half 128-column block
    cfg = synth.MoEConfig("f8pin", 31, T=T, H=H, E=E, k=2, I=I, w_dtype=fmt)
    q = synth.gen_experts(cfg)
    x = synth.gen_x(cfg)
    tok = np.repeat(np.arange(T), E)
    eid = np.tile(np.arange(E), T)
    y, h, hq = oracle.expert_rows_f8(x, q, I, tok, eid, want_h=True)
    gu, sgu, dn, sdn = _w8_matrices(q, fmt, E, H, I)
    xq, s = oracle.quantize_x(x)
    for r, (t, e) in enumerate(zip(tok, eid)):
        a = (xq[t] @ gu[e].T) * float(s[t]) * sgu[e]
        hh = oracle.format_op("round_bf16", a[:I] / (1 + np.exp(-a[:I])) * a[I:])
        np.testing.assert_allclose(h[r], hh, rtol=2.0 ** -8, atol=1e-12)
        # hq: each 128-block re-encoded with its power-of-two scale
        for b0 in range(0, I, 128):
            blk = h[r, b0:b0 + 128]
            eb = oracle.format_op("block_exp", [np.abs(blk).max()])[0]
            want = oracle.format_op("round_e4m3", blk * 2.0 ** -eb) * 2.0 ** eb
            assert np.array_equal(hq[r, b0:b0 + 128], want)
        np.testing.assert_allclose(y[r], (hq[r] @ dn[e].T) * sdn[e], rtol=1e-11, atol=1e-13)
    # the down stage alone, fed the same h, reproduces the rows
    assert np.array_equal(oracle.down_rows_f8(h, q, eid, H), y)


def test_f8_error_against_exact_path_is_small():
    """Statistical bound: the F8 encodings cost a few percent of the output RMS."""
    cfg = synth.MoEConfig("f8err", 32, T=8, H=256, E=4, k=2, I=256, w_dtype="fp8")
    q = synth.gen_experts(cfg)
    x = synth.gen_x(cfg)
    tok = np.repeat(np.arange(cfg.T), cfg.E)
    eid = np.tile(np.arange(cfg.E), cfg.T)
    y8 = oracle.expert_rows_f8(x, q, cfg.I, tok, eid)
    yw = oracle.expert_rows(x, q, cfg.I, tok, eid)
    rel = np.abs(y8 - yw).max() / np.sqrt(np.mean(yw ** 2))
    assert 1e-4 < rel < 0.25, rel
