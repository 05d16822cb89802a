"""GPU parity of the routed MoE layer against the CPU oracle (MI355X).

Every stage is checked on its own against the oracle fed the GPU's own
upstream outputs (router logits, selection, permute bit-exact, expert rows,
finalize), and the whole layer end to end against the oracle's layer. Small
configurations cover ragged and degenerate shapes in full; Beam-sized ones
(decode T=128, prefill T=16384 with Zipf load, NVFP4 T=4096, FP8) are checked
in full where the oracle is fast enough and on sampled rows otherwise, in the
launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import sparse_moe_layer_gemm_amd as moe
import synth
from tests.gpu_harness import (Layer, bits, check_experts, check_finalize, check_layer,
                               check_permute, check_router, forward_norm_vs_stages, log,
                               touched_bf16_experts)

pytestmark = pytest.mark.gpu

MC = synth.MoEConfig
SMALL = [
    synth.CONFIGS["tiny_fp32"],
    MC("ragged_bf16", 101, T=67, H=128, E=20, k=3, I=64),
    MC("k1", 102, T=40, H=256, E=16, k=1, I=128),
    MC("k_equals_E", 103, T=30, H=192, E=8, k=8, I=192),
    MC("crowded_experts", 104, T=600, H=256, E=4, k=2, I=128),
    MC("single_expert", 105, T=33, H=128, E=1, k=1, I=64),
    MC("zipf_bias_small", 106, T=200, H=256, E=32, k=4, I=128, zipf_s=1.1),
    MC("fp8_small", 107, T=50, H=256, E=8, k=2, I=128, w_dtype="fp8"),
    MC("fp4_small", 108, T=50, H=256, E=8, k=2, I=192, w_dtype="fp4"),
    MC("fp4_many_rows", 109, T=300, H=512, E=16, k=4, I=256, w_dtype="fp4"),
    # either side of the NVFP4 streaming / tiled boundary (more than 16 rows
    # per expert on average goes tiled): 16 rows per expert stream in 8-row
    # passes, 18 take the tiled kernels with short experts
    MC("fp4_stream_16rows", 140, T=64, H=512, E=16, k=4, I=256, w_dtype="fp4"),
    MC("fp4_tile_18rows", 141, T=72, H=512, E=16, k=4, I=256, w_dtype="fp4"),
    # ~12 rows per expert on wider products (I = 512, H = 1024): one to three
    # 8-row NVFP4 streaming passes per expert, 32 gate/up and 32 down column tiles
    MC("fp4_stream_12rows_wide", 142, T=48, H=1024, E=8, k=2, I=512, w_dtype="fp4"),
    MC("f32_ragged", 110, T=37, H=64, E=9, k=2, I=64, x_dtype="f32", w_dtype="f32"),
    # fp32 experts with many 16-row passes per expert
    MC("f32_many_rows", 130, T=300, H=256, E=4, k=2, I=192, x_dtype="f32", w_dtype="f32"),
    # >= 32 rows per expert: the 128 x 256 tiled kernel, with partial N tiles
    # (I = 192: second gate/up tile half valid; H = 192: down tile 3/4 valid)
    MC("tile_ragged", 112, T=150, H=192, E=4, k=2, I=192),
    MC("tile_zipf", 113, T=512, H=256, E=16, k=4, I=128, zipf_s=1.1),
    # quantised weights on the tiled kernels (>= 32 rows per expert): partial
    # N tiles on both tile shapes, Zipf load for a mix of 256- and 128-row tiles
    MC("fp8_tile", 114, T=200, H=256, E=8, k=4, I=192, w_dtype="fp8"),
    MC("fp4_tile_ragged", 115, T=150, H=192, E=4, k=2, I=192, w_dtype="fp4"),
    MC("fp4_tile_zipf", 116, T=512, H=256, E=16, k=4, I=128, zipf_s=1.1, w_dtype="fp4"),
    # ~150 rows per expert: an expert's last tile takes its tail of <= 32 rows
    # (tiles of 129 .. 160 rows, five row fragments)
    MC("fp4_merged_tail", 121, T=300, H=256, E=4, k=2, I=192, w_dtype="fp4"),
    MC("fp8_merged_tail", 122, T=300, H=192, E=4, k=2, I=128, w_dtype="fp8"),
    # fp8-MFMA mode (against the oracle's F8 encodings): few and many rows per
    # expert, partial N tiles and a partial 128-column h block (I = 192),
    # Zipf load for both tile shapes
    MC("f8_fp8_tile", 117, T=200, H=256, E=8, k=4, I=192, w_dtype="fp8", qmode="f8"),
    MC("f8_fp4_ragged", 118, T=150, H=192, E=4, k=2, I=192, w_dtype="fp4", qmode="f8"),
    MC("f8_fp4_zipf", 119, T=512, H=256, E=16, k=4, I=128, zipf_s=1.1, w_dtype="fp4", qmode="f8"),
    MC("f8_fp8_few_rows", 120, T=20, H=128, E=8, k=2, I=64, w_dtype="fp8", qmode="f8"),
    # fewer pairs than experts: the streaming grid runs over touched-expert
    # slots; K split for gate/up (4 splits bf16, 2 splits E2M1 / E4M3), a
    # K tail on the E2M1 down product (I = 192 is 1.5 super steps), partial
    # column slices (I = 320, H = 1024 / 2048)
    MC("few_pairs_split_bf16", 121, T=2, H=1024, E=64, k=3, I=320),
    MC("few_pairs_split_fp4", 122, T=3, H=2048, E=32, k=2, I=192, w_dtype="fp4"),
    MC("few_pairs_split_fp8", 123, T=3, H=1024, E=32, k=2, I=320, w_dtype="fp8"),
    # K split on the down product too (4 splits bf16, 2 E4M3), whose partial
    # sums moe_forward adds inside its finalize; H = 320 leaves the second
    # 256-column chunk of that finalize a quarter full
    MC("split_down_ragged_h", 124, T=2, H=320, E=16, k=4, I=1024),
    MC("split_down_fp8", 125, T=3, H=320, E=16, k=3, I=1024, w_dtype="fp8"),
    # one token: moe_forward's select kernel also writes the permute (every
    # expert chosen; k < E with E not a multiple of 64)
    MC("one_token_all_experts", 126, T=1, H=256, E=8, k=8, I=128),
    MC("one_token_k3", 127, T=1, H=192, E=70, k=3, I=64),
    # at most 32 pairs with gate/up split: the down kernel forms h in LDS from
    # the gate/up partial sums (here several rows per expert, down split too)
    MC("fold_h_32_pairs", 128, T=4, H=1024, E=16, k=8, I=1024),
    # h formed in the down kernel where its last K split is short (I = 1600:
    # 50 K steps in splits of 9, the last of 5), so that split's first items
    # span more than one row of h
    MC("fold_short_last_split", 129, T=2, H=2048, E=8, k=2, I=1600),
]


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype == torch.bfloat16:
        return np.array_equal(bits(a), bits(b))
    return torch.equal(a, b)


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_layer_parity(cfg):
    log(f"[parity] {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} w={cfg.w_dtype}")
    L = Layer(cfg)
    r = L.stages()
    rt = check_router(L, r)
    check_permute(L, r)
    ey = check_experts(L, r, np.arange(cfg.T * cfg.k))
    check_finalize(L, r)
    lay = check_layer(L, r, np.arange(cfg.T))
    f = L.forward()
    assert _same_bits(f["out"], r["out"]) and torch.equal(f["out_f32"], r["out_f32"])
    assert torch.equal(f["ids"], r["ids"]) and torch.equal(f["w"], r["w"])
    log(f"  logits {rt['logit_rel_err']:.2e} ambiguous {rt['ambiguous']} y {ey:.2e} "
        f"out {lay['out_rel_err']:.2e}")


def test_zero_tokens_is_a_noop():
    cfg = MC("empty", 111, T=0, H=128, E=8, k=2, I=64)
    L = Layer(cfg)
    f = L.forward()
    assert f["out"].numel() == 0


def test_router_beam_shape():
    cfg = synth.CONFIGS["router_t128"]
    log(f"[parity] {cfg.name}")
    L = Layer(cfg)
    r = L.route()
    torch.cuda.synchronize()
    rt = check_router(L, r)
    log(f"  logits rel err {rt['logit_rel_err']:.2e}, ambiguous tokens {rt['ambiguous']}/{rt['tokens']}")


# Batches of >= 1024 bf16 tokens take the router through three bf16 products on
# the tiled MFMA kernel (weights split exactly into hi/mid/lo bf16 planes); all
# logits are checked, with a ragged last M tile and, for E = 200, zero-padded
# expert columns.
@pytest.mark.parametrize("T,H,E,k", [(1300, 5120, 256, 8), (1030, 640, 200, 6)])
def test_router_split_bf16_full(T, H, E, k):
    cfg = MC(f"router_x3_t{T}_e{E}", 120 + E, T=T, H=H, E=E, k=k, I=64, router_only=True)
    log(f"[parity] {cfg.name}")
    L = Layer(cfg)
    r = L.route()
    torch.cuda.synchronize()
    rt = check_router(L, r)
    log(f"  logits rel err {rt['logit_rel_err']:.2e}, ambiguous tokens {rt['ambiguous']}/{rt['tokens']}")


# Above 16384 pairs the permute runs as histogram / scan / scatter kernels over
# many workgroups; ids with heavy ties, ragged segment ends, few and many experts.
@pytest.mark.parametrize("P,E", [(40000, 256), (16448, 7), (131072, 256)])
def test_permute_many_pairs_bit_exact(P, E):
    import oracle
    rng = np.random.default_rng(P + E)
    k = 8 if E >= 8 else 4
    T = P // k
    p = rng.zipf(1.3, size=(T, k)) % E  # skewed, so long runs of equal ids
    ids = p.astype(np.int32)
    d = torch.from_numpy(ids).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    log(f"[parity] permute P={T * k} E={E}")
    moe.moe_permute(d, E, counts, offsets, sp, pp)
    torch.cuda.synchronize()
    c, o, s, q = oracle.permute(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(sp.cpu().numpy(), s)
    assert np.array_equal(pp.cpu().numpy(), q)


@pytest.fixture(scope="module")
def decode_layer():
    cfg = synth.CONFIGS["decode_t128"]
    log(f"[setup] {cfg.name}: generating and uploading inputs")
    return Layer(cfg)


def test_decode_beam_full(decode_layer):
    L = decode_layer
    cfg = L.cfg
    log(f"[parity] {cfg.name}")
    r = L.stages()
    rt = check_router(L, r)
    counts = check_permute(L, r)
    ey = check_experts(L, r, np.arange(cfg.T * cfg.k))
    check_finalize(L, r)
    lay = check_layer(L, r, np.arange(cfg.T))
    f = L.forward()
    assert _same_bits(f["out"], r["out"]) and torch.equal(f["out_f32"], r["out_f32"])
    g = L.forward()  # run twice: bit-identical (no atomics, fixed reduction orders)
    assert torch.equal(g["out_f32"], f["out_f32"])
    forward_norm_vs_stages(L, r)  # the layer ending in the fused finalize + norms
    log(f"  touched experts {int((counts > 0).sum())}, max rows {int(counts.max())}; logits "
        f"{rt['logit_rel_err']:.2e}; ambiguous {rt['ambiguous']}; y {ey:.2e}; out(fp32) "
        f"{lay['out_rel_err']:.2e}; out(bf16) {lay['out_bf16_rel_err']:.2e} (floor {lay['bf16_floor']:.2e})")


def test_decode_single_token(decode_layer):
    cfg = decode_layer.cfg.with_(name="decode_t1", T=1)
    L = Layer(cfg, x=decode_layer.x[:1].copy())
    r = L.stages()
    check_router(L, r)
    check_permute(L, r)
    check_experts(L, r, np.arange(cfg.k))
    check_finalize(L, r)
    lay = check_layer(L, r, [0])
    f = L.forward()  # the down GEMM's split partial sums added inside the finalize
    assert _same_bits(f["out"], r["out"]) and torch.equal(f["out_f32"], r["out_f32"])
    log(f"  T=1 out {lay['out_rel_err']:.2e}")


@pytest.mark.parametrize("T", [2, 4, 8])
def test_decode_small_batches(decode_layer, T):
    """Few touched experts: the streaming kernels split K (several splits at
    T = 2 and 4, two for gate/up at T = 8) and a reduction forms h and y; up to
    32 pairs the down kernel forms h itself, and inside moe_forward y's
    reduction is folded into the finalize (both bit-identical)."""
    cfg = decode_layer.cfg.with_(name=f"decode_t{T}", T=T)
    L = Layer(cfg, x=decode_layer.x[:T].copy())
    r = L.stages()
    check_router(L, r)
    check_permute(L, r)
    ey = check_experts(L, r, np.arange(T * cfg.k))
    check_finalize(L, r)
    lay = check_layer(L, r, np.arange(T))
    f = L.forward()
    assert _same_bits(f["out"], r["out"]) and torch.equal(f["out_f32"], r["out_f32"])
    log(f"  T={T} y {ey:.2e} out {lay['out_rel_err']:.2e}")


@pytest.mark.parametrize("T", [1, 4, 32])
def test_decode_wide_experts(T):
    """Expert width I = 2560 (the width the published checkpoint sizes imply),
    at batch sizes that take the split-K path (T = 1, 4) and the plain one."""
    cfg = MC(f"decode_i2560_t{T}", 130 + T, T=T, H=5120, E=256, k=8, I=2560, router_only=True)
    R = Layer(cfg)
    touched = np.unique(R.route()["ids"].cpu().numpy())
    cfg = cfg.with_(router_only=False)
    L = Layer(cfg, x=R.x, weights=touched_bf16_experts(cfg, touched))
    r = L.stages()
    check_router(L, r)
    check_permute(L, r)
    # every row at T <= 4; at T = 32 a seeded sample of rows and tokens
    rng = np.random.default_rng(T)
    rows = np.arange(T * cfg.k) if T <= 4 else np.sort(rng.choice(T * cfg.k, 48, replace=False))
    tokens = np.arange(T) if T <= 4 else np.sort(rng.choice(T, 6, replace=False))
    ey = check_experts(L, r, rows)
    check_finalize(L, r)
    lay = check_layer(L, r, tokens)
    log(f"  I=2560 T={T} touched {touched.size}: y {ey:.2e} out {lay['out_rel_err']:.2e}")


def test_decode_token_permutation(decode_layer):
    """Permuting the tokens permutes the output rows (bit for bit: every token's
    arithmetic is independent of its position)."""
    L = decode_layer
    perm = np.random.default_rng(5).permutation(L.cfg.T)
    L2 = Layer(L.cfg, x=np.ascontiguousarray(L.x[perm]))
    a = L.forward()
    b = L2.forward()
    assert torch.equal(b["ids"], a["ids"][torch.from_numpy(perm).cuda()])
    assert torch.equal(b["out_f32"], a["out_f32"][torch.from_numpy(perm).cuda()])


def _sample_rows(counts: np.ndarray, offsets: np.ndarray, n_random: int, seed: int) -> np.ndarray:
    """First and last rows of the hottest, median and coldest non-empty experts, plus random rows."""
    rng = np.random.default_rng(seed)
    nz = np.nonzero(counts)[0]
    by = nz[np.argsort(counts[nz])]
    picks = {by[-1], by[-2], by[len(by) // 2], by[0]}
    rows = set()
    for e in picks:
        rows.update({int(offsets[e]), int(offsets[e + 1] - 1), int(offsets[e] + 31),
                     int(offsets[e] + 32)})
    rows = {r for r in rows if 0 <= r < offsets[-1]}
    rows.update(rng.choice(offsets[-1], n_random, replace=False).tolist())
    return np.array(sorted(rows))


def _spread_rows(counts: np.ndarray, offsets: np.ndarray, per_expert: int) -> np.ndarray:
    """Rows of every non-empty expert: up to per_expert evenly spaced ones (its first
    and last included), plus, for the hottest expert, the rows on each side of every
    128-row tile boundary and of the 31/32 boundary."""
    rows = set()
    for e in np.nonzero(counts)[0]:
        o0, c = int(offsets[e]), int(counts[e])
        rows.update((o0 + np.unique(np.linspace(0, c - 1, min(c, per_expert)).astype(np.int64))).tolist())
    e = int(np.argmax(counts))
    o0, c = int(offsets[e]), int(counts[e])
    for b in list(range(128, c, 128)) + [32]:
        rows.update(o0 + r for r in (b - 1, b) if 0 <= r < c)
    return np.array(sorted(rows), dtype=np.int64)


def test_prefill_zipf_wide():
    """The prefill layer (T = 16384, Zipf load, compact expert rows, the launch the
    benchmark times): router logits and selection on every token, expert rows of
    every expert (>= 4096 rows, tile and 31/32 boundaries of the hottest), finalize
    on every token, 1024 tokens end to end, and the layer ending in the fused
    finalize + norms on 512 tokens."""
    cfg = synth.CONFIGS["prefill_t16384_zipf"]
    log(f"[parity] {cfg.name}: generating inputs")
    L = Layer(cfg)
    r = L.stages()
    assert "y16" in r  # the prefill layer runs on compact rows, as moe_forward does
    rt = check_router(L, r)
    counts = check_permute(L, r)
    offsets = r["offsets"].cpu().numpy()
    rows = _spread_rows(counts, offsets, 16)
    assert len(rows) >= 4096
    ey = check_experts(L, r, rows)
    check_finalize(L, r)
    rng = np.random.default_rng(3)
    tok = np.sort(rng.choice(cfg.T, 1024, replace=False))
    lay = check_layer(L, r, tok)
    f = L.forward()
    assert torch.equal(f["out_f32"], r["out_f32"])
    forward_norm_vs_stages(L, r, tokens=tok[:512])
    log(f"  load max {int(counts.max())} median {int(np.median(counts))} min {int(counts.min())}; "
        f"logits {rt['logit_rel_err']:.2e}, ambiguous {rt['ambiguous']} of {rt['tokens']}; "
        f"y {ey:.2e} over {len(rows)} rows; out over {lay['checked']} tokens: fp32 "
        f"{lay['out_rel_err']:.3e}, bf16 {lay['out_bf16_rel_err']:.3e} (floor {lay['bf16_floor']:.3e})")


# grouped by weight format, so each format's weights are generated once; the
# decode sizes (T = 1, 2, 128) run the streaming kernels, T = 1 and 2 with K
# split. The NVFP4 layer (T = 4096) is checked end to end on 512 tokens in both
# modes, the rest on 64.
@pytest.mark.parametrize("wdt,T,qmode", [("fp4", 4096, "w"), ("fp4", 4096, "f8"), ("fp4", 128, "w"),
                                         ("fp4", 1, "w"), ("fp8", 1024, "w"), ("fp8", 1024, "f8"),
                                         ("fp8", 128, "w"), ("fp8", 2, "w")])
def test_quantised_beam_sampled(wdt, T, qmode):
    cfg = synth.CONFIGS["nvfp4_t4096"].with_(name=f"{wdt}_t{T}_{qmode}", w_dtype=wdt, T=T,
                                             qmode=qmode)
    log(f"[parity] {cfg.name}: generating inputs")
    L = Layer(cfg)
    r = L.stages()
    n_tok = 512 if T == 4096 else min(64, T)
    rng = np.random.default_rng(6)
    tok = np.sort(rng.choice(cfg.T, n_tok, replace=False))
    if T == 4096:
        check_router(L, r)
    else:
        check_router(L, r, rows=tok)
    counts = check_permute(L, r)
    offsets = r["offsets"].cpu().numpy()
    rows = (_spread_rows(counts, offsets, 2) if T == 4096
            else _sample_rows(counts, offsets, min(64, cfg.T * cfg.k), 7))
    ey = check_experts(L, r, rows)
    check_finalize(L, r, tokens=None if T == 4096 else tok)
    lay = check_layer(L, r, tok)
    log(f"  y {ey:.2e} over {len(rows)} rows; out over {lay['checked']} of {lay['tokens']} tokens: "
        f"fp32 {lay['out_rel_err']:.3e}, bf16 {lay['out_bf16_rel_err']:.3e} "
        f"(floor {lay['bf16_floor']:.3e}); ambiguous {lay['ambiguous']}"
        + (f", F8-ambiguous {lay['f8_ambiguous']}" if "f8_ambiguous" in lay else ""))


# Ids outside [0, E) (the router never emits them): the permute gives such a pair
# no row (pair_pos -1, sorted_pair -1 past the last expert's rows) and the
# finalize adds nothing for it; both permute paths (one workgroup up to 16384
# pairs, three kernels above).
@pytest.mark.parametrize("T,k,E", [(100, 4, 16), (5000, 8, 64)])
def test_permute_and_finalize_skip_invalid_ids(T, k, E):
    rng = np.random.default_rng(T)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.05
    ids[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, E + 3)
    P = T * k
    d = torch.from_numpy(ids).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.full((P,), 12345, dtype=torch.int32, device="cuda")
    pp = torch.full((P,), 12345, dtype=torch.int32, device="cuda")
    log(f"[parity] permute with {int(bad.sum())} invalid ids, P={P}")
    moe.moe_permute(d, E, counts, offsets, sp, pp)
    torch.cuda.synchronize()
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    order = sorted(np.nonzero(valid)[0].tolist(), key=lambda p: (flat[p], p))
    want_sp = np.full(P, -1, np.int32)
    want_sp[:len(order)] = order
    want_pp = np.full(P, -1, np.int32)
    want_pp[order] = np.arange(len(order))
    assert np.array_equal(counts.cpu().numpy(), np.bincount(flat[valid], minlength=E))
    assert int(offsets[-1]) == len(order)
    assert np.array_equal(sp.cpu().numpy(), want_sp)
    assert np.array_equal(pp.cpu().numpy(), want_pp)
    H = 256
    y = torch.randn((P, H), generator=torch.Generator("cuda").manual_seed(T), device="cuda")
    w = torch.rand((T, k), generator=torch.Generator("cuda").manual_seed(T + 1), device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.moe_finalize(y, pp, w, out)
    torch.cuda.synchronize()
    yh, wh, pph = y.cpu().numpy(), w.cpu().numpy(), pp.cpu().numpy().reshape(T, k)
    want = np.zeros((T, H), np.float32)
    for j in range(k):  # slot order, fp32, as the kernel sums
        use = pph[:, j] >= 0
        want[use] = np.float32(wh[use, j, None]) * yh[pph[use, j]] + want[use]
    assert np.allclose(out.cpu().numpy(), want, rtol=1e-6, atol=1e-6)


def _shift_nvfp4_scales(hw: dict, max_shift: int) -> dict:
    """The same NVFP4 weights with each matrix's block scales divided by 2^s and its
    per-expert scales multiplied by 2^s (s the largest shift up to max_shift that
    keeps every nonzero block scale a normal E4M3 value): identical dequantised
    values, block scales far below the 448 the usual recipe gives its largest."""
    import oracle
    e4 = oracle.format_op("e4m3", np.arange(256))
    out = dict(hw)
    for key, g in (("gate_up_scale", "gate_up_gscale"), ("down_scale", "down_gscale")):
        for shift in range(max_shift, 0, -1):
            v = e4[hw[key]] * 2.0 ** -shift
            codes = synth.encode_e4m3_table(v)
            if np.array_equal(e4[codes], v) and np.all((np.abs(v) >= 2.0 ** -6) | (v == 0)):
                break
        out[key] = codes
        out[g] = (hw[g].astype(np.float64) * 2.0 ** shift).astype(np.float32)
    return out


def test_f8_nvfp4_small_block_scales():
    """NVFP4 weights encoded with small block scales (gate/up <= 2^-3): the
    fp8-MFMA mode re-encodes each 32-deep K block with its own power of two, so
    the layer's output is bit-identical to that on the usually scaled encoding
    of the same weights, and meets the bound against the oracle."""
    import dataclasses
    cfg = MC("f8_fp4_small_scales", 141, T=300, H=256, E=8, k=4, I=192, w_dtype="fp4", qmode="f8")
    hw = synth.gen_experts(cfg)
    hs = _shift_nvfp4_scales(hw, 12)
    outs = []
    for w in (hw, hs):
        dw = dataclasses.replace(moe.experts_to_device(w), qmode=moe.MOE_QMODE_F8)
        L = Layer(cfg, weights=(w, dw))
        outs.append((L, L.stages()))
    (La, ra), (Lb, rb) = outs
    assert torch.equal(ra["out_f32"], rb["out_f32"]), "small block scales change the F8 output"
    check_experts(Lb, rb, np.arange(cfg.T * cfg.k))
    lay = check_layer(Lb, rb, np.arange(cfg.T))
    log(f"  small block scales: decision-matched {lay['decision_matched_rel_err']:.3e} over "
        f"{lay['checked']} tokens")
