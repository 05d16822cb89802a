"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each part of the oracle is checked against something it does not share code
with: format tables from the OCP specifications, exactly rounded sums
(math.fsum), a dense NumPy brute force, Python's sorted(), numpy matmul,
closed forms and invariants of the layer's definition.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ formats
def _golden(kind):
    with open(os.path.join(GOLDEN, "formats.json")) as f:
        return json.load(f)[kind]


@pytest.mark.parametrize("kind", ["e4m3", "e2m1", "bf16"])
def test_format_tables_match_spec(kind):
    rows = _golden(kind)
    codes = np.array([c for c, _ in rows], np.float64)
    got = oracle.format_op(kind, codes)
    for (code, want), g in zip(rows, got):
        if want == "nan":
            assert math.isnan(g), code
        else:
            assert g == want and math.copysign(1, g) == math.copysign(1, want), (code, g, want)


def test_all_e4m3_codes_monotone_and_symmetric():
    codes = np.arange(0, 127, dtype=np.float64)
    v = oracle.format_op("e4m3", codes)
    assert np.all(np.diff(v) > 0)  # positive codes are ordered by value
    neg = oracle.format_op("e4m3", codes + 128)
    assert np.array_equal(neg, -v)


def test_round_bf16_matches_torch_on_fp32_values():
    import torch
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-30,
                        rng.standard_normal(2000) * 1e30]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.format_op("round_bf16", v.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_single_rounding_on_doubles():
    rng = np.random.default_rng(8)
    v = rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))
    # exact midpoints between bf16 neighbours and points a hair off them
    base = brute.round_bf16_bits_method(rng.standard_normal(3000))
    e = np.floor(np.log2(np.abs(base)))
    ulp = 2.0 ** (e - 7)
    mids = base + ulp / 2
    v = np.concatenate([v, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    got = oracle.format_op("round_bf16", v)
    want = brute.round_bf16_bits_method(v)
    assert np.array_equal(got, want)


def test_round_f32_is_nearest_even():
    rng = np.random.default_rng(9)
    v = rng.standard_normal(10000) * 1e3
    assert np.array_equal(oracle.format_op("round_f32", v), v.astype(np.float32).astype(np.float64))


# ------------------------------------------------------------------ router
def test_logits_exact_against_fsum():
    rng = np.random.default_rng(1)
    T, H, E = 5, 96, 7
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = (rng.standard_normal((H, E)) / np.sqrt(H)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.logits(x, wr, b)
    xf = brute.bf16_bits_to_f64(x)
    for t in range(T):
        for e in range(E):
            want = math.fsum([float(b[e])] + [xf[t, h] * float(wr[h, e]) for h in range(H)])
            assert abs(got[t, e] - want) <= 1e-14 * max(1.0, abs(want))


def test_logits_rows_subset_and_fp32_input():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 64)).astype(np.float32)
    wr = rng.standard_normal((64, 5)).astype(np.float32)
    full = oracle.logits(x, wr)
    np.testing.assert_allclose(full, x.astype(np.float64) @ wr.astype(np.float64), rtol=1e-13, atol=1e-13)
    sub = oracle.logits(x, wr, rows=[8, 0, 3])
    assert np.array_equal(sub, full[[8, 0, 3]])


# ------------------------------------------------------------------ routing
def _brute_route(v, k):
    T, E = v.shape
    p = np.exp(v - v.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ids = np.empty((T, k), np.int64)
    w = np.empty((T, k))
    for t in range(T):
        o = np.lexsort((np.arange(E), -v[t]))[:k]
        ids[t], w[t] = o, p[t, o] / p[t, o].sum()
    return ids, w


@pytest.mark.parametrize("E,k", [(256, 8), (32, 4), (9, 9), (5, 1), (64, 8)])
def test_route_matches_brute_sort(E, k):
    rng = np.random.default_rng(E * 10 + k)
    lg = rng.standard_normal((300, E))
    ids, w = oracle.route(lg, k, "bf16")
    bi, bw = _brute_route(brute.round_bf16_bits_method(lg), k)
    assert np.array_equal(ids, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-13, atol=1e-15)
    # invariants: k distinct ids in range, weights sum to one, descending order
    assert all(len(set(r)) == k for r in ids)
    assert ids.min() >= 0 and ids.max() < E
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_route_ties_go_to_lowest_id():
    # bf16 rounding collapses distinct logits onto one value: ties must order by id
    lg = np.zeros((3, 16))
    lg[0, [3, 7, 11]] = 1.0
    lg[1, :] = 0.5
    lg[2, [15, 2]] = [2.0 + 2 ** -12, 2.0]  # equal once rounded to bf16
    ids, w = oracle.route(lg, 4, "bf16")
    assert ids[0].tolist() == [3, 7, 11, 0]
    assert ids[1].tolist() == [0, 1, 2, 3]
    np.testing.assert_allclose(w[1], 0.25)
    assert ids[2].tolist()[:2] == [2, 15]
    np.testing.assert_allclose(w[2, 0], w[2, 1])


def test_route_k1_and_k_equals_E():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 12))
    ids, w = oracle.route(lg, 1, "f32")
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(lg.astype(np.float32), axis=1))
    ids, w, sel = oracle.route(lg, 12, "f32", want_sel=True)
    p = np.exp(sel - sel.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    full = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, full, rtol=1e-13)


def test_route_weights_equal_softmax_over_selected():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((40, 64)) * 3
    ids, w, sel = oracle.route(lg, 8, "bf16", want_sel=True)
    s = np.take_along_axis(sel, ids.astype(np.int64), axis=1)
    q = np.exp(s - s.max(1, keepdims=True))
    np.testing.assert_allclose(w, q / q.sum(1, keepdims=True), rtol=1e-13)


# ------------------------------------------------------------------ permute
@pytest.mark.parametrize("T,k,E", [(0, 8, 256), (1, 8, 256), (37, 4, 32), (500, 8, 256), (64, 1, 3)])
def test_permute_matches_sorted(T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32).reshape(T, k)
    counts, offsets, sp, pp = oracle.permute(ids, E)
    flat = ids.ravel()
    want = sorted(range(T * k), key=lambda p: (flat[p], p))
    assert sp.tolist() == want
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == T * k
    assert np.array_equal(pp[sp], np.arange(T * k))


def test_permute_rejects_out_of_range_ids():
    with pytest.raises(RuntimeError):
        oracle.permute(np.array([[0, 5]], np.int32), 4)


# ------------------------------------------------------------------ experts
def _tiny_experts(rng, E, H, I, dtype="bf16"):
    gu = (rng.standard_normal((E, H, 2 * I)) / np.sqrt(H)).astype(np.float32)
    dn = (rng.standard_normal((E, I, H)) / np.sqrt(I)).astype(np.float32)
    if dtype == "bf16":
        return {"dtype": "bf16", "gate_up": synth.f32_to_bf16_bits(gu), "down": synth.f32_to_bf16_bits(dn)}
    return {"dtype": "f32", "gate_up": gu, "down": dn}


def test_expert_rows_match_numpy_matmul():
    rng = np.random.default_rng(5)
    T, H, I, E = 10, 64, 32, 4
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ex = _tiny_experts(rng, E, H, I)
    tok = np.array([0, 3, 9, 9, 5])
    eid = np.array([1, 0, 3, 2, 1])
    y, h = oracle.expert_rows(x, ex, I, tok, eid, want_h=True)
    xf = brute.bf16_bits_to_f64(x)
    gu = brute.bf16_bits_to_f64(ex["gate_up"])
    dn = brute.bf16_bits_to_f64(ex["down"])
    for r, (t, e) in enumerate(zip(tok, eid)):
        a = xf[t] @ gu[e]
        hh = a[:I] / (1 + np.exp(-a[:I])) * a[I:]
        np.testing.assert_allclose(h[r], hh, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(y[r], hh @ dn[e], rtol=1e-11, atol=1e-13)


def _exact_quantised_case(rng, E, H, I, fmt):
    """f32 weights built from values the format represents exactly, and their encoding."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])  # E2M1 magnitudes (OCP MX v1.0)

    def fp4_matrix(N, K):
        mag = grid[rng.integers(0, 8, (N, K))]
        sign = np.where(rng.random((N, K)) < 0.5, -1.0, 1.0)
        sb_exp = rng.integers(-4, 3, (N, K // 16))  # block scales: powers of two
        g = 2.0 ** int(rng.integers(-6, -2))  # global scale: a power of two
        w = sign * mag * np.repeat(2.0 ** sb_exp, 16, axis=1) * g
        q = synth.pack_nibbles(synth.encode_e2m1(sign * mag))
        sb = synth.encode_e4m3(2.0 ** sb_exp)
        return w, q, sb, np.float32(g)

    def fp8_matrix(N, K):
        v = synth._E4M3_POS[rng.integers(0, 127, (N, K))] * np.where(rng.random((N, K)) < .5, -1, 1)
        s = (2.0 ** rng.integers(-8, -2, N)).astype(np.float32)
        return v * s[:, None].astype(np.float64), synth.encode_e4m3(v), s

    gu_f, dn_f = np.empty((E, H, 2 * I)), np.empty((E, I, H))
    q = {"dtype": fmt}
    parts = {k: [] for k in ["gate_up", "gate_up_scale", "gate_up_gscale", "down", "down_scale", "down_gscale"]}
    for e in range(E):
        if fmt == "fp4":
            w, qq, sb, g = fp4_matrix(2 * I, H)
            gu_f[e] = w.T
            parts["gate_up"].append(qq), parts["gate_up_scale"].append(sb), parts["gate_up_gscale"].append(g)
            w, qq, sb, g = fp4_matrix(H, I)
            dn_f[e] = w.T
            parts["down"].append(qq), parts["down_scale"].append(sb), parts["down_gscale"].append(g)
        else:
            w, qq, s = fp8_matrix(2 * I, H)
            gu_f[e] = w.T
            parts["gate_up"].append(qq), parts["gate_up_scale"].append(s)
            w, qq, s = fp8_matrix(H, I)
            dn_f[e] = w.T
            parts["down"].append(qq), parts["down_scale"].append(s)
    for key, v in parts.items():
        if v:
            q[key] = np.ascontiguousarray(np.stack(v))
    f32 = {"dtype": "f32", "gate_up": gu_f.astype(np.float32), "down": dn_f.astype(np.float32)}
    assert np.array_equal(f32["gate_up"].astype(np.float64), gu_f)  # exactly representable
    return q, f32


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_quantised_decode_is_exact(fmt):
    """Weights chosen on the format's grid: the quantised path must equal the fp32 path bit for bit."""
    rng = np.random.default_rng(11)
    T, H, I, E = 6, 64, 32, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    q, f32 = _exact_quantised_case(rng, E, H, I, fmt)
    tok = np.repeat(np.arange(T), E)
    eid = np.tile(np.arange(E), T)
    yq = oracle.expert_rows(x, q, I, tok, eid)
    yf = oracle.expert_rows(x, f32, I, tok, eid)
    assert np.array_equal(yq, yf)


def test_pack_nibbles_low_nibble_is_even_k():
    codes = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    assert synth.pack_nibbles(codes).tolist() == [[0x21, 0x43, 0x0F]]


# ------------------------------------------------------------------ finalize
def test_finalize_closed_form():
    rng = np.random.default_rng(6)
    T, k, H = 20, 4, 8
    P = T * k
    ys = np.repeat(np.arange(P, dtype=np.float32)[:, None], H, axis=1)  # row r is r * ones
    pp = rng.permutation(P).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = oracle.finalize(ys, pp, w, k)
    want = (w.astype(np.float64) * pp.reshape(T, k)).sum(1)
    np.testing.assert_allclose(out, np.repeat(want[:, None], H, axis=1), rtol=1e-15)


# ------------------------------------------------------------------ whole layer
def _dense_inputs(cfg, rng=None):
    x = synth.gen_x(cfg)
    wr, b = synth.gen_router(cfg)
    ex = synth.gen_experts(cfg)
    xf = x.astype(np.float64) if cfg.x_dtype == "f32" else brute.bf16_bits_to_f64(x)
    if ex["dtype"] == "f32":
        gu, dn = ex["gate_up"].astype(np.float64), ex["down"].astype(np.float64)
    else:
        gu, dn = brute.bf16_bits_to_f64(ex["gate_up"]), brute.bf16_bits_to_f64(ex["down"])
    return x, wr, b, ex, xf, gu, dn


@pytest.mark.parametrize("cfg", [
    synth.CONFIGS["tiny_fp32"],
    synth.MoEConfig("tiny_bf16", 21, T=40, H=128, E=16, k=4, I=64),
    synth.MoEConfig("tiny_bf16_k8", 22, T=33, H=64, E=64, k=8, I=64),
    synth.MoEConfig("tiny_bias", 23, T=50, H=64, E=20, k=3, I=32, zipf_s=1.1),
])
def test_layer_matches_dense_brute_force(cfg):
    x, wr, b, ex, xf, gu, dn = _dense_inputs(cfg)
    sel = cfg.logits_dtype
    got = oracle.layer(x, wr, b, ex, cfg.I, cfg.k, sel)
    want = brute.dense_layer(xf, wr, b, gu, dn, cfg.k, sel)
    assert np.array_equal(got["ids"], want["ids"])
    np.testing.assert_allclose(got["w"], want["w"], rtol=1e-12)
    scale = np.sqrt(np.mean(want["out"] ** 2))
    assert np.max(np.abs(got["out"] - want["out"])) <= 1e-12 * scale


def test_layer_token_permutation_invariance():
    cfg = synth.MoEConfig("perm", 31, T=24, H=64, E=8, k=2, I=32)
    x, wr, b, ex, *_ = _dense_inputs(cfg)
    perm = np.random.default_rng(0).permutation(cfg.T)
    a = oracle.layer(x, wr, b, ex, cfg.I, cfg.k)
    c = oracle.layer(np.ascontiguousarray(x[perm]), wr, b, ex, cfg.I, cfg.k)
    assert np.array_equal(c["out"], a["out"][perm])
    assert np.array_equal(c["ids"], a["ids"][perm])


def test_identical_experts_reduce_to_one_ffn():
    """With every expert equal, the renormalised mixture is that expert's SwiGLU FFN
    (the dense-MLP layers of the model are this FFN)."""
    cfg = synth.MoEConfig("same", 41, T=16, H=64, E=16, k=4, I=32)
    x = synth.gen_x(cfg)
    wr, _ = synth.gen_router(cfg)
    one = synth.gen_experts(cfg.with_(E=1))
    ex = {"dtype": "bf16", "gate_up": np.repeat(one["gate_up"], cfg.E, 0),
          "down": np.repeat(one["down"], cfg.E, 0)}
    got = oracle.layer(x, wr, None, ex, cfg.I, cfg.k)["out"]
    want = brute.swiglu_ffn(brute.bf16_bits_to_f64(x), brute.bf16_bits_to_f64(one["gate_up"][0]),
                            brute.bf16_bits_to_f64(one["down"][0]))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_single_expert_layer_is_ffn():
    cfg = synth.MoEConfig("e1", 42, T=12, H=64, E=1, k=1, I=32, x_dtype="f32", w_dtype="f32")
    x, wr, b, ex, xf, gu, dn = _dense_inputs(cfg)
    got = oracle.layer(x, wr, None, ex, cfg.I, 1, "f32")
    assert np.all(got["w"] == 1.0) and np.all(got["ids"] == 0)
    np.testing.assert_allclose(got["out"], brute.swiglu_ffn(xf, gu[0], dn[0]), rtol=1e-12, atol=1e-13)


def test_layer_rows_subset_equals_full():
    cfg = synth.MoEConfig("rows", 43, T=30, H=64, E=8, k=2, I=32)
    x, wr, b, ex, *_ = _dense_inputs(cfg)
    full = oracle.layer(x, wr, b, ex, cfg.I, cfg.k)
    rows = [29, 3, 3, 17]
    sub = oracle.layer(x, wr, b, ex, cfg.I, cfg.k, rows=rows)
    assert np.array_equal(sub["out"], full["out"][rows])
