"""ctypes wrapper of the plain CPU oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package. The GPU library neither imports nor links it, and it imports
nothing from the GPU package.

All results are float64 numpy arrays (ids and permutation arrays int32).
Inputs are numpy arrays in their storage formats: x float32 or bf16 bits
(uint16), router weights float32, expert weights as produced by
``synth.gen_experts``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

DT = {"f32": 0, "bf16": 1, "fp8": 2, "fp4": 3}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP) into liboracle.so."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wno-unknown-pragmas", SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check(rc, fn):
    if rc != 0:
        raise RuntimeError(f"oracle {fn} failed with code {rc}")


def _rows(rows):
    if rows is None:
        return None
    return np.ascontiguousarray(rows, dtype=np.int64)


def _xdt(x):
    if x.dtype == np.float32:
        return DT["f32"]
    if x.dtype == np.uint16:
        return DT["bf16"]
    raise TypeError(f"x must be float32 or bf16 bits (uint16), got {x.dtype}")


def format_op(kind: str, values) -> np.ndarray:
    """Format decoding/rounding of the oracle: kind in bf16, e4m3, e2m1 (codes -> value),
    round_bf16, round_f32, round_e4m3 (value -> rounded value), block_exp (amax -> the
    power-of-two block exponent of the fp8-MFMA mode)."""
    k = {"bf16": 0, "e4m3": 1, "e2m1": 2, "round_bf16": 3, "round_f32": 4, "round_e4m3": 5,
         "block_exp": 6}[kind]
    v = np.ascontiguousarray(values, dtype=np.float64).ravel()
    out = np.empty_like(v)
    f = lib().oracle_format
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    _check(f(k, _p(v), v.size, _p(out)), "format")
    return out.reshape(np.shape(values))


def logits(x, w_router, bias=None, rows=None) -> np.ndarray:
    """Exact router logits [n, E] (float64)."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    wr = np.ascontiguousarray(w_router, dtype=np.float32)
    E = wr.shape[1]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r = _rows(rows)
    n = T if r is None else r.size
    out = np.empty((n, E), np.float64)
    f = lib().oracle_logits
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    _check(f(_xdt(x), _p(x), T, H, _p(wr), _p(b), E, _p(r), n, _p(out)), "logits")
    return out


def route(logits_, k: int, sel_dtype: str = "bf16", want_sel: bool = False):
    """(ids [n,k] int32, w [n,k] float64[, sel [n,E]]) from logits [n,E]."""
    lg = np.ascontiguousarray(logits_, dtype=np.float64)
    n, E = lg.shape
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    sel = np.empty((n, E), np.float64) if want_sel else None
    f = lib().oracle_route
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    _check(f(DT[sel_dtype], _p(lg), n, E, k, _p(ids), _p(w), _p(sel)), "route")
    return (ids, w, sel) if want_sel else (ids, w)


def permute(ids, E: int):
    """(counts [E], offsets [E+1], sorted_pair [T*k], pair_pos [T*k]) int32."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    pp = np.empty(T * k, np.int32)
    f = lib().oracle_permute
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 4
    _check(f(_p(ids), T, k, E, _p(counts), _p(offsets), _p(sp), _p(pp)), "permute")
    return counts, offsets, sp, pp


def _wargs(experts: dict):
    dt = DT[experts["dtype"]]
    arr = lambda key: (None if experts.get(key) is None else np.ascontiguousarray(experts[key]))
    gu, dn = arr("gate_up"), arr("down")
    gus, dns = arr("gate_up_scale"), arr("down_scale")
    gug, dng = arr("gate_up_gscale"), arr("down_gscale")
    keep = (gu, dn, gus, dns, gug, dng)
    return dt, keep


def expert_rows(x, experts: dict, I: int, tokens, expert_ids, want_h: bool = False):
    """y [n, H] (and h [n, I]) for the (token, expert) rows given."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    dt, (gu, dn, gus, dns, gug, dng) = _wargs(experts)
    E = gu.shape[0]
    tok = np.ascontiguousarray(tokens, dtype=np.int32).ravel()
    ex = np.ascontiguousarray(expert_ids, dtype=np.int32).ravel()
    n = tok.size
    y = np.empty((n, H), np.float64)
    h = np.empty((n, I), np.float64) if want_h else None
    f = lib().oracle_expert_rows
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int] + [ctypes.c_void_p] * 8 + [ctypes.c_int64] + [ctypes.c_void_p] * 2
    _check(f(_xdt(x), _p(x), T, H, I, E, dt, _p(gu), _p(dn), _p(gus), _p(dns), _p(gug), _p(dng),
             _p(tok), _p(ex), n, _p(y), _p(h)), "expert_rows")
    return (y, h) if want_h else y


def expert_rows_f8(x, experts: dict, I: int, tokens, expert_ids, want_h: bool = False):
    """F8 mode (fp8-MFMA encodings, see oracle.c): y [n, H], and with want_h also
    h [n, I] (bf16-rounded) and hq [n, I] (dequantised E4M3 codes times 2^e)."""
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("F8 mode takes bf16 activations")
    T, H = x.shape
    dt, (gu, dn, gus, dns, gug, dng) = _wargs(experts)
    E = gu.shape[0]
    tok = np.ascontiguousarray(tokens, dtype=np.int32).ravel()
    ex = np.ascontiguousarray(expert_ids, dtype=np.int32).ravel()
    n = tok.size
    y = np.empty((n, H), np.float64)
    h = np.empty((n, I), np.float64) if want_h else None
    hq = np.empty((n, I), np.float64) if want_h else None
    f = lib().oracle_expert_rows_f8
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int] + [ctypes.c_void_p] * 8 + [ctypes.c_int64] + [ctypes.c_void_p] * 3
    _check(f(_p(x), T, H, I, E, dt, _p(gu), _p(dn), _p(gus), _p(dns), _p(gug), _p(dng),
             _p(tok), _p(ex), n, _p(y), _p(h), _p(hq)), "expert_rows_f8")
    return (y, h, hq) if want_h else y


def down_rows_f8(h, experts: dict, expert_ids, H: int):
    """F8 down stage on given h rows (bf16 values [n, I]): y [n, H]."""
    h = np.ascontiguousarray(h, dtype=np.float64)
    n, I = h.shape
    dt, (gu, dn, gus, dns, gug, dng) = _wargs(experts)
    E = gu.shape[0]
    ex = np.ascontiguousarray(expert_ids, dtype=np.int32).ravel()
    y = np.empty((n, H), np.float64)
    f = lib().oracle_down_rows_f8
    f.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_int] + [ctypes.c_void_p] * 7 + [ctypes.c_int64] + [ctypes.c_void_p] * 2
    _check(f(H, I, E, dt, _p(gu), _p(dn), _p(gus), _p(dns), _p(gug), _p(dng), _p(ex), n, _p(h), _p(y)),
           "down_rows_f8")
    return y


def quantize_x(x):
    """F8-mode activation quantisation: (E4M3 values [T, H], fp32 scales [T])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T, H = x.shape
    xq = np.empty((T, H), np.float64)
    s = np.empty(T, np.float32)
    f = lib().oracle_quantize_x
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    _check(f(_p(x), T, H, _p(xq), _p(s)), "quantize_x")
    return xq, s


def finalize(y_sorted, pair_pos, w, k: int, rows=None) -> np.ndarray:
    """out [n, H] (float64) = slot-ordered weighted sum of the fp32 sorted expert rows."""
    ys = np.ascontiguousarray(y_sorted, dtype=np.float32)
    pp = np.ascontiguousarray(pair_pos, dtype=np.int32).ravel()
    ww = np.ascontiguousarray(w, dtype=np.float32).ravel()
    H = ys.shape[1]
    T = pp.size // k
    r = _rows(rows)
    n = T if r is None else r.size
    out = np.empty((n, H), np.float64)
    f = lib().oracle_finalize
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    _check(f(_p(ys), _p(pp), _p(ww), T, k, H, _p(r), n, _p(out)), "finalize")
    return out


def rms_norm(v, gamma, eps: float) -> np.ndarray:
    """RMSNorm of each row in float64: v / sqrt(mean(v^2) + eps) * gamma."""
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=1, keepdims=True) + eps) * g


def finalize_norm(y_sorted, pair_pos, w, k: int, residual_bits, gamma_post_bits,
                  gamma_next_bits, eps: float, rows=None) -> dict:
    """MoE finalize fused with the sandwich post-norm, the residual add and the
    next sublayer's pre-norm (vLLM PR #61978, Status table row #62366: the
    fused all-reduce "with Beam's sandwich norms and MoE finalize"; the pages
    do not define the norm, so these are conventions: RMSNorm with weight
    gamma and epsilon eps, bf16 residual stream and bf16 norm weights):

        m      = finalize(y_sorted, pair_pos, w)          (slot-ordered sum)
        post   = m / sqrt(mean(m^2) + eps) * gamma_post
        r      = RNE_bf16(residual + post)                (the new residual)
        normed = RNE_bf16(r / sqrt(mean(r^2) + eps) * gamma_next)

    Everything in float64 on the bf16 / fp32 inputs; the next norm reads the
    rounded residual, as the next sublayer would. Returns m, post, r and
    normed (float64 values; r and normed are bf16-representable)."""
    m = finalize(y_sorted, pair_pos, w, k, rows=rows)
    res = format_op("bf16", np.asarray(residual_bits))
    if rows is not None:
        res = res[np.asarray(rows)]
    gp = format_op("bf16", np.asarray(gamma_post_bits))
    gn = format_op("bf16", np.asarray(gamma_next_bits))
    post = rms_norm(m, gp, eps)
    r = format_op("round_bf16", res + post)
    normed = format_op("round_bf16", rms_norm(r, gn, eps))
    return {"m": m, "post": post, "r": r, "normed": normed}


def layer(x, w_router, bias, experts: dict, I: int, k: int, sel_dtype: str = "bf16", rows=None,
          qmode: str = "w"):
    """Whole layer for the given tokens: dict(out [n,H], ids [n,k], w [n,k], logits [n,E]).
    qmode "w": quantised weights dequantised exactly, bf16 activations; "f8": fp8-MFMA mode."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    wr = np.ascontiguousarray(w_router, dtype=np.float32)
    E = wr.shape[1]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    dt, (gu, dn, gus, dns, gug, dng) = _wargs(experts)
    r = _rows(rows)
    n = T if r is None else r.size
    out = np.empty((n, H), np.float64)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    lg = np.empty((n, E), np.float64)
    f = lib().oracle_layer_q
    f.argtypes = ([ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_int32] * 4 +
                  [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 7 +
                  [ctypes.c_int64] + [ctypes.c_void_p] * 4)
    _check(f({"w": 0, "f8": 1}[qmode], _xdt(x), _p(x), T, H, I, E, k, _p(wr), _p(b), DT[sel_dtype],
             dt, _p(gu), _p(dn), _p(gus), _p(dns), _p(gug), _p(dng), _p(r), n, _p(out), _p(ids),
             _p(w), _p(lg)), "layer")
    return {"out": out, "ids": ids, "w": w, "logits": lg}
