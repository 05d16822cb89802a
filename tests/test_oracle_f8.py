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


def _covering_exponent(m):
    """Smallest integer e with 448 * 2^e >= m (0 for m = 0), by direct search."""
    m = np.asarray(m, dtype=np.float64)
    e = np.where(m > 0, np.floor(np.log2(np.where(m > 0, m, 1.0))) - 9, 0).astype(np.int64)
    for _ in range(3):  # the estimate is within one or two of the answer
        e = np.where((m > 0) & (448.0 * np.ldexp(1.0, e) < m), e + 1, e)
    for _ in range(3):
        e = np.where((m > 0) & (448.0 * np.ldexp(1.0, e - 1) >= m), e - 1, e)
    return e


def _w8_matrices(q, fmt, E, H, I):
    """The operand values of the F8 mode, built from the format tables and the
    generator's table-driven E4M3 encoder (not the oracle's rounding): gate/up
    [E, 2I, H] and down [E, H, I] (K-major rows), and the column scales. NVFP4
    codes are re-encoded per 32-deep K block with 2^-s, s = (the exponent field
    of the block's larger E4M3 scale) - 12, and multiplied back by 2^s."""
    e4 = oracle.format_op("e4m3", np.arange(256))
    e2 = oracle.format_op("e2m1", np.arange(16))

    def mat(codes, scales, gsc, N, K):
        if fmt == "fp8":
            return e4[codes.reshape(E, N, K)], scales.astype(np.float64)
        lo, hi = codes & 15, codes >> 4
        nib = np.stack([lo, hi], -1).reshape(E, N, K)
        sv = e4[scales.reshape(E, N, K // 16)]
        mag = (scales.reshape(E, N, K // 32, 2) & 0x7F).astype(np.int64)
        sig = np.repeat((mag.max(axis=3) >> 3) - 12, 32, axis=2)
        # the shift keeps every product on the E4M3 grid's normal range unsaturated
        assert np.all(6.0 * np.abs(np.repeat(sv, 16, axis=2)) * np.ldexp(1.0, -sig) < 448.0)
        prod = e2[nib] * np.repeat(sv, 16, axis=2) * np.ldexp(1.0, -sig)
        v = e4[synth.encode_e4m3_table(prod)] * np.ldexp(1.0, sig)
        return v, np.repeat(gsc.astype(np.float64)[:, None], N, axis=1)

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


def test_covering_exponent_matches_block_exp():
    m = np.concatenate([6.0 * oracle.format_op("e4m3", np.arange(127)), [0.0, 448.0, 449.0, 2688.0]])
    assert np.array_equal(_covering_exponent(m), oracle.format_op("block_exp", m).astype(np.int64))


def _small_scale_copy(q, max_shift):
    """The same NVFP4 weights with every block scale of a matrix divided by 2^s and
    its per-expert scales multiplied by 2^s: identical dequantised values (powers
    of two), block scales far below the 448 the usual recipe gives its largest.
    s is the largest shift up to max_shift that keeps every nonzero scale a
    normal E4M3 value (exactly representable, exponent field shifted by s)."""
    e4 = oracle.format_op("e4m3", np.arange(256))
    out = dict(q)
    for key, g in (("gate_up_scale", "gate_up_gscale"), ("down_scale", "down_gscale")):
        for shift in range(max_shift, 0, -1):
            v = e4[q[key]] * 2.0 ** -shift
            codes = synth.encode_e4m3_table(v)
            if np.array_equal(e4[codes], v) and np.all((np.abs(v) >= 2.0 ** -6) | (v == 0)):
                break
        out[key] = codes
        out[g] = (q[g].astype(np.float64) * 2.0 ** shift).astype(np.float32)
    return out


def test_f8_nvfp4_small_block_scales():
    """NVFP4 weights whose gate/up block scales are all <= 2^-3 (the usual recipe
    puts the largest at 448): the exact dequantisation is unchanged, and the F8
    mode's per-block re-encoding gives the same rows as with the usual scales
    (the re-encoded products keep full E4M3 precision whatever the scales'
    range), so its error against the exact path is the same; a fixed shift
    would not."""
    cfg = synth.MoEConfig("f8small", 33, T=8, H=256, E=3, k=2, I=256, w_dtype="fp4")
    q = synth.gen_experts(cfg)
    qs = _small_scale_copy(q, 12)
    e4 = oracle.format_op("e4m3", np.arange(256))
    assert np.abs(e4[qs["gate_up_scale"]]).max() <= 2.0 ** -3
    x = synth.gen_x(cfg)
    tok = np.repeat(np.arange(cfg.T), cfg.E)
    eid = np.tile(np.arange(cfg.E), cfg.T)
    yw = oracle.expert_rows(x, q, cfg.I, tok, eid)
    assert np.array_equal(oracle.expert_rows(x, qs, cfg.I, tok, eid), yw)
    y8 = oracle.expert_rows_f8(x, q, cfg.I, tok, eid)
    y8s = oracle.expert_rows_f8(x, qs, cfg.I, tok, eid)
    rms = np.sqrt(np.mean(yw ** 2))
    eps, eps_s = np.abs(y8 - yw).max() / rms, np.abs(y8s - yw).max() / rms
    np.testing.assert_allclose(y8s, y8, rtol=0, atol=1e-9 * rms)
    # a fixed shift of 2^-3 for every block (the largest any NVFP4 block needs)
    # would push these products into E4M3 subnormals: the gate/up sums on
    # operands re-encoded that way move far more
    e4 = oracle.format_op("e4m3", np.arange(256))
    e2 = oracle.format_op("e2m1", np.arange(16))
    xq, st = oracle.quantize_x(x)

    def gate_up_sums(qq, fixed):
        codes = qq["gate_up"]
        nib = np.stack([codes & 15, codes >> 4], -1).reshape(cfg.E, 2 * cfg.I, cfg.H)
        sv = np.repeat(e4[qq["gate_up_scale"]], 16, axis=2)
        if fixed:
            w8 = e4[synth.encode_e4m3_table(e2[nib] * sv / 8.0)] * 8.0
        else:
            w8 = _w8_matrices(qq, "fp4", cfg.E, cfg.H, cfg.I)[0]
        g = qq["gate_up_gscale"].astype(np.float64)[:, None, None]
        return np.stack([xq[t] @ (w8[e] * g[e]).T * st[t] for t, e in zip(tok, eid)])

    a_usual = gate_up_sums(q, False)
    a_small = gate_up_sums(qs, False)
    a_fixed = gate_up_sums(qs, True)
    r = np.sqrt(np.mean(a_usual ** 2))
    d_small = np.abs(a_small - a_usual).max() / r
    d_fixed = np.abs(a_fixed - a_usual).max() / r
    print(f"F8 vs exact NVFP4 rows: usual scales {eps:.3e}, scales <= 2^-3 {eps_s:.3e}; gate/up sums "
          f"moved by the scale change: per-block shift {d_small:.1e}, fixed 2^-3 shift {d_fixed:.1e}")
    assert d_small < 1e-12 and d_fixed > 1e-2
