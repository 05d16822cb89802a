"""Shared helpers of the GPU parity tests: upload seeded inputs, run the layer
through the C ABI stage by stage, and compare with the oracle.

Tolerances (fixed by the layer's statement of parity, readings in the tests):
  - router logits: max_e |l_gpu - l_ref| <= 1e-5 * scale per token, scale = the
    row's max |l_ref| (no less than the RMS of the batch's logits);
  - expert ids: bit-exact, except tokens whose ranking a 1e-5 relative change
    of the logits could alter (counted and reported);
  - outputs: max |out_gpu - out_ref| / rms(out_ref) <= 2e-2 (bf16 experts),
    3e-2 (FP8), 6e-2 (NVFP4), 1e-4 (all-fp32 layer).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
import sparse_moe_layer_gemm_amd as moe
import synth

DEV = "cuda"
TOL_OUT = {"bf16": 2e-2, "fp8": 3e-2, "fp4": 6e-2, "f32": 1e-4}
LOGIT_REL = 1e-5

_weight_cache: dict = {}


def log(msg: str):
    print(msg, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_experts(cfg: synth.MoEConfig) -> dict:
    key = (cfg.weight_seed if cfg.weight_seed is not None else cfg.seed, cfg.w_dtype, cfg.E, cfg.H, cfg.I)
    if key not in _weight_cache:
        _weight_cache.clear()  # keep one layer's weights at a time
        hostw = synth.gen_experts(cfg)
        _weight_cache[key] = (hostw, moe.experts_to_device(hostw, DEV))
    hostw, dw = _weight_cache[key]
    if cfg.qmode == "f8":
        dw = dataclasses.replace(dw, qmode=moe.MOE_QMODE_F8)
    return hostw, dw


def touched_bf16_experts(cfg: synth.MoEConfig, touched) -> tuple:
    """bf16 expert weights of which only the `touched` experts are generated.

    Host: full [E, ...] arrays (untouched slices are never written, so they
    stay unbacked zero pages); device: full [E, ...] tensors whose untouched
    slices are left uninitialised. Only routed experts are ever read, by the
    kernels and by the oracle, so this stands in for the whole layer at a
    fraction of the generation cost.
    """
    assert cfg.w_dtype == "bf16"
    touched = np.asarray(sorted(set(int(e) for e in touched)))
    sub = synth.gen_experts(cfg, experts=touched)
    E, H, I = cfg.E, cfg.H, cfg.I
    hw = {"dtype": "bf16", "gate_up": np.empty((E, H, 2 * I), np.uint16),
          "down": np.empty((E, I, H), np.uint16)}
    hw["gate_up"][touched] = sub["gate_up"]
    hw["down"][touched] = sub["down"]
    gu = torch.empty((E, H, 2 * I), dtype=torch.bfloat16, device=DEV)
    dn = torch.empty((E, I, H), dtype=torch.bfloat16, device=DEV)
    idx = torch.from_numpy(touched).to(DEV)
    gu[idx] = torch.from_numpy(sub["gate_up"].view(np.int16)).to(DEV).view(torch.bfloat16)
    dn[idx] = torch.from_numpy(sub["down"].view(np.int16)).to(DEV).view(torch.bfloat16)
    return hw, moe.ExpertWeights(moe.MOE_BF16, gu, dn)


class Layer:
    """Seeded inputs of one configuration, on the host and on the device."""

    def __init__(self, cfg: synth.MoEConfig, x: np.ndarray | None = None, weights=None):
        self.cfg = cfg
        self.x = synth.gen_x(cfg) if x is None else x
        self.wr, self.bias = synth.gen_router(cfg)
        if cfg.x_dtype == "f32":
            self.dx = torch.from_numpy(self.x).to(DEV)
        else:
            self.dx = moe.to_device_bf16(self.x, DEV)
        self.dwr = torch.from_numpy(self.wr).to(DEV)
        self.dbias = None if self.bias is None else torch.from_numpy(self.bias).to(DEV)
        if weights is not None:
            self.hw, self.dw = weights
        elif not cfg.router_only:
            self.hw, self.dw = host_experts(cfg)

    @property
    def ldt(self):
        return moe.MOE_F32 if self.cfg.x_dtype == "f32" else moe.MOE_BF16

    def route(self):
        c = self.cfg
        T, E, k = c.T, c.E, c.k
        tdt = torch.float32 if c.x_dtype == "f32" else torch.bfloat16
        r = {"logits": torch.empty((T, E), dtype=tdt, device=DEV),
             "logits_f32": torch.empty((T, E), dtype=torch.float32, device=DEV),
             "ids": torch.empty((T, k), dtype=torch.int32, device=DEV),
             "w": torch.empty((T, k), dtype=torch.float32, device=DEV)}
        ws = moe.workspace(moe.moe_route_workspace_size(T, c.H, E))
        moe.moe_route(self.dx, self.dwr, self.dbias, k, self.ldt, r["logits"], r["logits_f32"],
                      r["ids"], r["w"], ws)
        return r

    def stages(self):
        """route -> permute -> experts -> finalize, each through its own entry point."""
        c = self.cfg
        T, H, E, k, I = c.T, c.H, c.E, c.k, c.I
        r = self.route()
        P = T * k
        r["counts"] = torch.empty(E, dtype=torch.int32, device=DEV)
        r["offsets"] = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        r["sorted_pair"] = torch.empty(P, dtype=torch.int32, device=DEV)
        r["pair_pos"] = torch.empty(P, dtype=torch.int32, device=DEV)
        moe.moe_permute(r["ids"], E, r["counts"], r["offsets"], r["sorted_pair"], r["pair_pos"])
        ws = moe.workspace(moe.moe_experts_workspace_size(T, H, I, E, k, self.dw))
        r["experts_ws"] = ws
        r["out"] = torch.empty((T, H), dtype=self.dx.dtype, device=DEV)
        r["out_f32"] = torch.empty((T, H), dtype=torch.float32, device=DEV)
        # compact expert rows wherever the library supports them (as moe_forward
        # does); the checks then see the exactly decoded fp32 rows
        y16 = torch.empty((P, H), dtype=torch.int16, device=DEV)
        ysc = torch.empty((P, H // 64), dtype=torch.uint8, device=DEV)
        try:
            moe.moe_experts_rows16(self.dx, I, E, k, r["offsets"], r["sorted_pair"], self.dw, y16,
                                   ysc, ws)
            r["y16"], r["y16_scale"] = y16, ysc
            r["y"] = rows16_decode(y16, ysc)
            moe.moe_finalize_rows16(y16, ysc, r["pair_pos"], r["w"], r["out"], r["out_f32"])
        except moe.MoEError as err:
            if err.status != 2:  # MOE_ERR_UNSUPPORTED: the fp32 rows
                raise
            del y16, ysc
            r["y"] = torch.empty((P, H), dtype=torch.float32, device=DEV)
            moe.moe_experts(self.dx, I, E, k, r["offsets"], r["sorted_pair"], self.dw, r["y"], ws)
            moe.moe_finalize(r["y"], r["pair_pos"], r["w"], r["out"], r["out_f32"])
        torch.cuda.synchronize()
        return r

    def forward(self):
        c = self.cfg
        T, H, E, k, I = c.T, c.H, c.E, c.k, c.I
        f = {"out": torch.empty((T, H), dtype=self.dx.dtype, device=DEV),
             "out_f32": torch.empty((T, H), dtype=torch.float32, device=DEV),
             "ids": torch.empty((T, k), dtype=torch.int32, device=DEV),
             "w": torch.empty((T, k), dtype=torch.float32, device=DEV)}
        ws = moe.workspace(moe.moe_forward_workspace_size(T, H, I, E, k, self.dw))
        moe.moe_forward(self.dx, self.dwr, self.dbias, self.dw, I, k, f["out"], ws,
                        out_f32=f["out_f32"], topk_ids=f["ids"], topk_w=f["w"])
        torch.cuda.synchronize()
        return f


def rows16_decode(y16: torch.Tensor, y16_scale: torch.Tensor) -> torch.Tensor:
    """Compact expert rows -> fp32 rows: fp16 value times 2^(scale byte - 127),
    one scale per row and 64-column block (exact in fp32)."""
    v = y16.view(torch.float16).float()
    e = y16_scale.to(torch.int32) - 127
    return torch.ldexp(v, e.repeat_interleave(64, dim=1).float())


# ------------------------------------------------------------------ comparisons
def round_sel(values: np.ndarray, sel: str) -> np.ndarray:
    if sel == "bf16":
        return oracle.format_op("round_bf16", values)
    return values.astype(np.float32).astype(np.float64)


def logit_scale(lref: np.ndarray) -> np.ndarray:
    """Per-token scale of the 1e-5 logit tolerance: the row's largest |logit|, but no
    less than the RMS of all logits of the batch (a row of one or two experts can
    cancel to a tiny logit whose fp32 rounding error is set by its terms, not by it)."""
    rms = float(np.sqrt(np.mean(lref ** 2))) if lref.size else 0.0
    return np.maximum(np.abs(lref).max(axis=1), rms)


def ambiguous_tokens(lref: np.ndarray, k: int, sel: str, rel: float = LOGIT_REL) -> np.ndarray:
    """Tokens whose top-k set or order a relative logit change of `rel` could alter.

    (i) the exact gap between the k-th and (k+1)-th logit is below rel, or
    (ii) with d = rel * (the token's logit scale), some adjacent pair (a before b) among the first
    k + 1 in selection order has (round(l_a - d), -a) <= (round(l_b + d), -b).
    """
    n, E = lref.shape
    ids = np.broadcast_to(np.arange(E), (n, E))
    v = round_sel(lref, sel)
    order = np.lexsort((ids, -v), axis=-1)
    d = rel * logit_scale(lref)[:, None]
    lo = round_sel(lref - d, sel)
    hi = round_sel(lref + d, sel)
    amb = np.zeros(n, dtype=bool)
    ex = np.sort(lref, axis=1)[:, ::-1]
    if k < E:
        amb |= (ex[:, k - 1] - ex[:, k]) < rel
    m = min(k + 1, E)
    rows = np.arange(n)
    for i in range(m - 1):
        a, b = order[:, i], order[:, i + 1]
        la, hb = lo[rows, a], hi[rows, b]
        amb |= (la < hb) | ((la == hb) & (a > b))
    return amb


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(got.astype(np.float64) - ref))) / max(rms, 1e-30)


def check_router(layer: Layer, r: dict, rows=None) -> dict:
    """Logits vs the exact oracle logits; selection vs oracle on the GPU's own logits."""
    c = layer.cfg
    sel = c.logits_dtype
    lref = oracle.logits(layer.x, layer.wr, layer.bias, rows=rows)
    lf = r["logits_f32"].cpu().numpy().astype(np.float64)
    if rows is not None:
        lf = lf[rows]
    scale = logit_scale(lref)
    worst = float(np.max(np.abs(lf - lref).max(axis=1) / scale))
    assert worst <= LOGIT_REL, f"logits rel err {worst}"
    # emitted logits are the rounding of the fp32 sums
    if sel == "bf16":
        lb = oracle.format_op("bf16", bits(r["logits"]).astype(np.float64))
        if rows is not None:
            lb = lb[rows]
        assert np.array_equal(lb, oracle.format_op("round_bf16", lf.astype(np.float32).astype(np.float64)))
    else:
        lb = r["logits"].cpu().numpy().astype(np.float64)
        if rows is not None:
            lb = lb[rows]
        assert np.array_equal(lb, lf)
    # stage-isolated selection: oracle routing on the GPU's own emitted logits, no exceptions
    ids = r["ids"].cpu().numpy()
    w = r["w"].cpu().numpy()
    if rows is not None:
        ids, w = ids[rows], w[rows]
    oid, ow = oracle.route(lb, c.k, sel)
    assert np.array_equal(ids, oid), "selection on the GPU's logits differs from the oracle's"
    assert np.max(np.abs(w - ow)) <= 2e-6
    assert np.allclose(w.sum(1), 1.0, atol=1e-5)
    # end to end: routing of the exact logits, ambiguous tokens excepted
    rid, _ = oracle.route(lref, c.k, sel)
    amb = ambiguous_tokens(lref, c.k, sel)
    mism = np.any(ids != rid, axis=1)
    assert not np.any(mism & ~amb), f"{int(np.sum(mism & ~amb))} unambiguous tokens routed differently"
    return {"logit_rel_err": worst, "ambiguous": int(amb.sum()), "ambiguous_mismatched": int(mism.sum()),
            "tokens": len(ids), "lref": lref, "amb": amb}


def check_permute(layer: Layer, r: dict):
    ids = r["ids"].cpu().numpy()
    counts, offsets, sp, pp = oracle.permute(ids, layer.cfg.E)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["sorted_pair"].cpu().numpy(), sp)
    assert np.array_equal(r["pair_pos"].cpu().numpy(), pp)
    return counts


# ------------------------------------------------------------------ h and the fp8-MFMA mode
def gpu_h(r: dict, P: int, I: int) -> np.ndarray:
    """The kernel's bf16 h [P, I] (sorted rows): moe_experts leaves it at the
    start of its workspace."""
    ws = r["experts_ws"]
    hb = ws[:P * I * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(P, I)
    return oracle.format_op("bf16", hb.astype(np.float64))


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid just above |v| (8 significant bits); 2^-133 at 0."""
    a = np.abs(v)
    _, ex = np.frexp(a)  # a = m 2^ex, 0.5 <= m < 1
    return np.where(a > 0, np.ldexp(1.0, ex - 8), np.ldexp(1.0, -133))


def h_tol(href: np.ndarray) -> np.ndarray:
    """How far the kernel's bf16 h may sit from the oracle's: one bf16 step (the
    rounding of an fp32 value within fp32 error of the exact one), or 2^-12 of
    the row's largest |h| where a near-cancelling gate or up sum leaves a tiny h
    whose fp32 accumulation error (set by the size of the summed terms, not by
    the sum) exceeds a step of that value. Measured on the fp8-MFMA kernels:
    at most 2.5e-5 of the row maximum, a tenth of this floor."""
    return np.maximum(bf16_ulp(href), 2.0 ** -12 * np.abs(href).max(axis=1, keepdims=True))


def check_h_rows(hg: np.ndarray, href: np.ndarray, what: str):
    """Every element of the kernel's h within h_tol of the oracle's."""
    d = np.abs(hg - href)
    bad = d > h_tol(href)
    assert not bad.any(), (f"{what}: {int(bad.sum())} h values beyond one bf16 step of the oracle's "
                           f"(worst {float(d.max()):.3e})")


def f8_h_codes(h: np.ndarray, I: int):
    """The oracle's E4M3 encoding of bf16 h rows [n, I] in the fp8-MFMA mode: per
    128-column block the exponent e of the block's amax (block_exp) and codes
    RNE_e4m3(h 2^-e). Returns (codes times 2^e [n, I], block exponents [n, nb])."""
    n = h.shape[0]
    nb = (I + 127) // 128
    eb = np.empty((n, nb), np.int64)
    hq = np.empty_like(h)
    for b in range(nb):
        sl = slice(128 * b, min(128 * (b + 1), I))
        e = oracle.format_op("block_exp", np.abs(h[:, sl]).max(axis=1)).astype(np.int64)
        eb[:, b] = e
        hq[:, sl] = np.ldexp(oracle.format_op("round_e4m3", np.ldexp(h[:, sl], -e[:, None])),
                             e[:, None])
    return hq, eb


def e4m3_spacing(a: np.ndarray) -> np.ndarray:
    """Spacing of the E4M3 grid just above magnitude a (scaled domain): 2^-9 below
    the smallest normal 2^-6, else 2^(floor(log2 a) - 3)."""
    _, ex = np.frexp(a)
    return np.where(a >= 2.0 ** -6, np.ldexp(1.0, ex - 4), 2.0 ** -9)


def f8_decisions(hg: np.ndarray, hr: np.ndarray, I: int, what: str):
    """E4M3 decisions of the fp8-MFMA mode taken on the kernel's h (hg) against
    those taken on the oracle's h (hr), both bf16 [n, I] and within h_tol of each
    other (check_h_rows). A code may differ only as a rounding-boundary decision:
      - the block exponent differs by one (the two block maxima straddle a
        power-of-two threshold of the block scale), or
      - under the same exponent, the codes are ordered as the two h values and
        the rounding midpoint between the oracle's code and its grid neighbour
        towards the kernel's code lies between the two h values; where the two
        h are within one bf16 step the codes must also be neighbours on the
        E4M3 grid (only a near-cancelled tiny h, within the fp32 floor of
        h_tol, may move across more than one grid step).
    Any other difference fails. Returns (rows touched by a boundary decision
    [n] bool, differing codes, differing block exponents)."""
    qg, eg = f8_h_codes(hg, I)
    qr, er = f8_h_codes(hr, I)
    within = np.abs(hg - hr) <= h_tol(hr)
    n = hg.shape[0]
    touched = np.zeros(n, bool)
    n_code = n_blk = 0
    unexplained = 0
    for b in range(eg.shape[1]):
        sl = slice(128 * b, min(128 * (b + 1), I))
        blk = eg[:, b] != er[:, b]
        unexplained += int(np.sum(blk & (np.abs(eg[:, b] - er[:, b]) != 1)))
        n_blk += int(blk.sum())
        touched |= blk
        diff = (qg[:, sl] != qr[:, sl]) & ~blk[:, None]
        if not diff.any():
            continue
        e = er[:, b][:, None]
        vg, vr = np.ldexp(hg[:, sl], -e), np.ldexp(hr[:, sl], -e)
        cg, cr = np.ldexp(qg[:, sl], -e), np.ldexp(qr[:, sl], -e)
        up = cg > cr
        # grid neighbour of the oracle's code towards the kernel's: away from zero
        # the spacing above |cr|, towards zero the spacing below it
        away = (cr == 0) | ((cr > 0) == up)
        a = np.abs(cr)
        step = np.where(away, e4m3_spacing(a), e4m3_spacing(np.nextafter(a, 0.0)))
        nb = np.where(up, cr + step, cr - step)
        mid = (cr + nb) / 2
        ordered = (cg - cr) * (vg - vr) > 0
        straddle = (np.minimum(vg, vr) <= mid) & (mid <= np.maximum(vg, vr))
        one_step = np.abs(hg[:, sl] - hr[:, sl]) <= bf16_ulp(hr[:, sl])
        ok = within[:, sl] & ordered & straddle & ((cg == nb) | ~one_step)
        unexplained += int(np.sum(diff & ~ok))
        n_code += int(diff.sum())
        touched |= diff.any(axis=1)
    assert unexplained == 0, f"{what}: {unexplained} E4M3 h decisions differ without a rounding boundary"
    return touched, n_code, n_blk


def check_experts(layer: Layer, r: dict, rows: np.ndarray) -> float:
    """Sorted rows y[r] vs the oracle's FFN of (token, expert) of that row, and the
    kernel's h of those rows vs the oracle's."""
    c = layer.cfg
    P = c.T * c.k
    sp = r["sorted_pair"].cpu().numpy()
    ids = r["ids"].cpu().numpy().ravel()
    rows = np.asarray(rows, dtype=np.int64)
    pairs = sp[rows]
    idx = torch.from_numpy(rows).to(DEV)
    y = r["y"].index_select(0, idx).cpu().numpy()
    hg = gpu_h(r, P, c.I)[rows] if c.x_dtype == "bf16" else None
    if c.qmode == "f8":
        yref, href, hqref = oracle.expert_rows_f8(layer.x, layer.hw, c.I, pairs // c.k, ids[pairs],
                                                  want_h=True)
        # the harness's encoding helper reproduces the oracle's own codes
        assert np.array_equal(f8_h_codes(href, c.I)[0], hqref)
        check_h_rows(hg, href, "gate/up h (fp8 MFMA)")
        touched, n_code, n_blk = f8_decisions(hg, href, c.I, "sampled rows")
        # the down stage with the decisions taken on the kernel's own h
        ydown = oracle.down_rows_f8(hg, layer.hw, ids[pairs], c.H)
        err = rel_err(y, ydown)
        # rows no boundary decision touched: against the oracle end to end
        keep = ~touched
        err_e2e = rel_err(y[keep], yref[keep]) if keep.any() else 0.0
        log(f"  f8: {n_code} h codes and {n_blk} block exponents decided across a rounding "
            f"boundary ({int(touched.sum())} of {len(rows)} rows); y on the kernel's h {err:.3e}, "
            f"y end to end (other rows) {err_e2e:.3e}, all rows {rel_err(y, yref):.3e}")
        assert err_e2e <= TOL_OUT[c.w_dtype], f"expert rows rel err {err_e2e} (no boundary decision)"
    else:
        yref, href = oracle.expert_rows(layer.x, layer.hw, c.I, pairs // c.k, ids[pairs], want_h=True)
        if hg is not None:
            check_h_rows(hg, href, "gate/up h")
        err = rel_err(y, yref)
    assert err <= TOL_OUT[c.w_dtype], f"expert rows rel err {err}"
    return err


def check_finalize(layer: Layer, r: dict, tokens=None) -> float:
    """Finalize vs the oracle's weighted sum of the GPU's own rows, and bf16 = RNE(fp32)."""
    c = layer.cfg
    pp = r["pair_pos"].cpu().numpy()
    w = r["w"].cpu().numpy()
    if tokens is None:
        y = r["y"].cpu().numpy()
        ref = oracle.finalize(y, pp, w, c.k)
        got = r["out_f32"].cpu().numpy()
    else:
        tokens = np.asarray(tokens, dtype=np.int64)
        need = np.unique(pp.reshape(c.T, c.k)[tokens].ravel())
        ysub = r["y"].index_select(0, torch.from_numpy(need).to(DEV)).cpu().numpy()
        remap = np.full(c.T * c.k, -1, np.int64)
        remap[need] = np.arange(len(need))
        pp_sub = remap[pp.reshape(c.T, c.k)[tokens]].astype(np.int32)
        ref = oracle.finalize(ysub, pp_sub.ravel(), w[tokens], c.k)
        got = r["out_f32"].cpu().numpy()[tokens]
    err = rel_err(got, ref)
    assert err <= 1e-5, f"finalize rel err {err}"
    outf = r["out_f32"].cpu().numpy()
    if c.x_dtype == "bf16":
        want = torch.from_numpy(outf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(bits(r["out"]), want), "bf16 output is not RNE of the fp32 output"
    else:
        assert np.array_equal(r["out"].cpu().numpy(), outf)
    return err


def layer_ref_f8(layer: Layer, tokens: np.ndarray) -> dict:
    """The oracle's fp8-MFMA-mode layer for the given tokens, composed of its
    steps (logits, routing, expert rows, slot-ordered weighted sum: the order
    oracle.layer sums in) so that the rows' h is available too."""
    c = layer.cfg
    lref = oracle.logits(layer.x, layer.wr, layer.bias, rows=tokens)
    ids, w = oracle.route(lref, c.k, c.logits_dtype)
    y, h, _ = oracle.expert_rows_f8(layer.x, layer.hw, c.I, np.repeat(tokens, c.k), ids.ravel(),
                                    want_h=True)
    y = y.reshape(len(tokens), c.k, c.H)
    out = np.zeros((len(tokens), c.H))
    for j in range(c.k):
        out += w[:, j, None] * y[:, j]
    return {"out": out, "ids": ids, "w": w, "logits": lref, "h": h.reshape(len(tokens), c.k, c.I)}


def check_layer(layer: Layer, r: dict, tokens, amb_all=None) -> dict:
    """End to end: GPU fp32 output vs the oracle's layer, on tokens whose routing
    a 1e-5 change of the logits cannot alter.

    In the fp8-MFMA mode every E4M3 decision on h that differs between the
    kernel and the oracle must be a rounding-boundary decision (f8_decisions);
    the tokens such a decision touches are counted as F8-ambiguous. Then
      - every token no boundary decision touched meets the bound against the
        oracle's layer;
      - every token meets the bound against the decision-matched oracle layer:
        the oracle's down stage on the kernel's h, i.e. the oracle's own codes
        except at the boundary decisions, summed with the oracle's weights;
      - at Beam width (I >= 1024), where one decision moves an output by a small
        fraction of the bound, every token also meets it against the oracle's
        layer as it stands."""
    c = layer.cfg
    tokens = np.asarray(tokens, dtype=np.int64)
    f8 = {}
    if c.qmode == "f8":
        ref = layer_ref_f8(layer, tokens)
    else:
        ref = oracle.layer(layer.x, layer.wr, layer.bias, layer.hw, c.I, c.k, c.logits_dtype,
                           rows=tokens, qmode=c.qmode)
    amb = ambiguous_tokens(ref["logits"], c.k, c.logits_dtype)
    keep = ~amb
    outf = r["out_f32"].cpu().numpy()[tokens]
    tol = TOL_OUT[c.w_dtype]
    if c.qmode == "f8" and keep.any():
        # the kernel's h of each checked token's k rows, against the oracle's
        pp = r["pair_pos"].cpu().numpy().reshape(c.T, c.k)[tokens]
        hg = gpu_h(r, c.T * c.k, c.I)[pp.ravel()]
        ids = r["ids"].cpu().numpy()[tokens]
        assert np.all(np.all(ids == ref["ids"], axis=1) | amb)
        rk = np.repeat(keep, c.k)
        hr = ref["h"].reshape(-1, c.I)
        check_h_rows(hg[rk], hr[rk], "gate/up h of the checked tokens")
        touched, n_code, n_blk = f8_decisions(hg[rk], hr[rk], c.I, "checked tokens")
        f8_amb = np.zeros(len(tokens), bool)
        f8_amb[np.nonzero(keep)[0]] = touched.reshape(-1, c.k).any(axis=1)
        # decision-matched reference: the oracle's down stage on the kernel's h
        yd = oracle.down_rows_f8(hg[rk], layer.hw, ref["ids"][keep].ravel(), c.H)
        yd = yd.reshape(-1, c.k, c.H)
        out_dm = np.zeros((int(keep.sum()), c.H))
        for j in range(c.k):
            out_dm += ref["w"][keep, j, None] * yd[:, j]
        err_dm = rel_err(outf[keep], out_dm)
        clean = keep & ~f8_amb
        err_clean = rel_err(outf[clean], ref["out"][clean]) if clean.any() else None
        f8 = {"f8_ambiguous": int(f8_amb.sum()), "f8_codes": n_code, "f8_block_exps": n_blk,
              "decision_matched_rel_err": err_dm, "clean_rel_err": err_clean,
              "clean_tokens": int(clean.sum())}
        log(f"  f8 layer: {n_code} h codes / {n_blk} block exponents on a rounding boundary; "
            f"{f8['f8_ambiguous']} of {int(keep.sum())} tokens F8-ambiguous; decision-matched "
            f"{err_dm:.3e} (all), end to end {err_clean if err_clean is None else f'{err_clean:.3e}'} "
            f"({f8['clean_tokens']} untouched tokens)")
        assert err_dm <= tol, f"decision-matched layer output rel err {err_dm}"
        if err_clean is not None:
            assert err_clean <= tol, f"layer output rel err {err_clean} (tokens without boundary decisions)"
    err = rel_err(outf[keep], ref["out"][keep]) if keep.any() else 0.0
    out_bits = bits(r["out"])[tokens] if c.x_dtype == "bf16" else None
    lit = None
    if out_bits is not None and keep.any():
        ob = oracle.format_op("bf16", out_bits.astype(np.float64))
        lit = rel_err(ob[keep], ref["out"][keep])
        floor = rel_err(oracle.format_op("round_bf16", ref["out"][keep]), ref["out"][keep])
    else:
        floor = None
    if c.qmode != "f8" or c.I >= 1024:
        assert err <= tol, f"layer output rel err {err}"
    return {"out_rel_err": err, "out_bf16_rel_err": lit, "bf16_floor": floor,
            "ambiguous": int(amb.sum()), "tokens": len(tokens), "checked": int(keep.sum()), **f8}


# ------------------------------------------------------------------ finalize + norms
NORM_REL = 1e-5


def norm_inputs(seed: int, T: int, H: int):
    """Seeded bf16 residual [T, H] and norm weights [H] (bits) for the fused finalize + norms."""
    rng = np.random.default_rng([seed, T, H])
    res = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gp = synth.f32_to_bf16_bits((0.5 + rng.random(H)).astype(np.float32))
    gn = synth.f32_to_bf16_bits((0.5 + rng.random(H)).astype(np.float32))
    return res, gp, gn


def to_bf16_dev(bits_u16) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def bracket(got, exact, d):
    """got (bf16 values) lies between RNE(v - d) and RNE(v + d); returns the mask of
    elements where those two differ (rounding-boundary cases)."""
    lo = oracle.format_op("round_bf16", exact - d)
    hi = oracle.format_op("round_bf16", exact + d)
    bad = (got < lo) | (got > hi)
    assert not bad.any(), f"{int(bad.sum())} values outside the rounding bracket"
    return lo != hi


def check_norm_outputs(y, pp, w, k, res, gp, gn, eps, r_bits, n_bits, what=""):
    """The fused finalize + norms' outputs (bf16 bits) against the oracle's
    finalize_norm on the same fp32 expert rows y, positions pp and weights w.

    The residual is checked against the oracle's exact pre-rounding value v =
    residual + post: it must lie between RNE(v - d) and RNE(v + d), d = 1e-5 x
    the row's max |v| (the sum can cancel, so fp32 error is absolute at the row's
    scale), and must equal the oracle's rounded residual wherever those two
    agree. The next sublayer's input is checked from the oracle's norm u of the
    kernel's own residual, d = 1e-5 |u| per element (a product), and must equal
    RNE(u) wherever the bracket is one value."""
    ref = oracle.finalize_norm(y, pp, w, k, res, gp, gn, eps)
    v = oracle.format_op("bf16", res) + ref["post"]
    r = oracle.format_op("bf16", r_bits)
    edge_r = bracket(r, v, NORM_REL * np.max(np.abs(v), axis=1, keepdims=True))
    assert np.all((r == ref["r"]) | edge_r), "residual differs from the oracle's off a rounding boundary"
    gnv = oracle.format_op("bf16", gn)
    u = oracle.rms_norm(r, gnv, eps)
    n = oracle.format_op("bf16", n_bits)
    edge_n = bracket(n, u, NORM_REL * np.abs(u))
    assert np.all((n == oracle.format_op("round_bf16", u)) | edge_n)
    flips_r = int(np.sum(r != ref["r"]))
    flips_n = int(np.sum(n != oracle.format_op("round_bf16", u)))
    log(f"finalize_norm{what} T={w.shape[0]} H={y.shape[1]} k={k}: {flips_r} residual and "
        f"{flips_n} normed values round the other way (at a rounding boundary)")
    return flips_r, flips_n


def forward_norm_vs_stages(layer: Layer, r: dict, eps: float = 1e-6, tokens=None, seed: int = 0):
    """moe_forward_norm against the stage-by-stage layer (r, from Layer.stages) followed
    by moe_finalize_norm on the same rows (bit for bit: the same kernels and sums), and
    against the oracle's finalize_norm on the layer's own rows (all tokens, or `tokens`)."""
    c = layer.cfg
    T, H = c.T, c.H
    res, gp, gn = norm_inputs(seed + c.seed, T, H)
    dres, dgp, dgn = to_bf16_dev(res), to_bf16_dev(gp), to_bf16_dev(gn)
    r_out, n_out = torch.empty_like(dres), torch.empty_like(dres)
    ws = moe.workspace(moe.moe_forward_workspace_size(T, H, c.I, c.E, c.k, layer.dw))
    ids = torch.empty((T, c.k), dtype=torch.int32, device=DEV)
    moe.moe_forward_norm(layer.dx, layer.dwr, layer.dbias, layer.dw, c.I, c.k, dres, dgp, dgn, eps,
                         r_out, n_out, ws, topk_ids=ids)
    s_r, s_n = torch.empty_like(dres), torch.empty_like(dres)
    if "y16" in r:
        moe.moe_finalize_norm_rows16(r["y16"], r["y16_scale"], r["pair_pos"], r["w"], dres, dgp,
                                     dgn, eps, s_r, s_n)
    else:
        moe.moe_finalize_norm(r["y"], r["pair_pos"], r["w"], dres, dgp, dgn, eps, s_r, s_n)
    torch.cuda.synchronize()
    assert torch.equal(ids, r["ids"])
    assert np.array_equal(bits(r_out), bits(s_r)) and np.array_equal(bits(n_out), bits(s_n)), \
        "moe_forward_norm differs from the stages + moe_finalize_norm"
    pp = r["pair_pos"].cpu().numpy().reshape(T, c.k)
    w = r["w"].cpu().numpy()
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    need = np.unique(pp[tokens].ravel())
    ysub = r["y"].index_select(0, torch.from_numpy(need).to(DEV)).cpu().numpy()
    remap = np.full(T * c.k, -1, np.int64)
    remap[need] = np.arange(len(need))
    return check_norm_outputs(ysub, remap[pp[tokens]].astype(np.int32).ravel(), w[tokens], c.k,
                              res[tokens], gp, gn, eps, bits(r_out)[tokens], bits(n_out)[tokens],
                              what=f" via moe_forward_norm ({c.name})")
