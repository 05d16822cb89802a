"""Dense NumPy brute force of the routed MoE layer, for tiny shapes only.

An implementation independent of the oracle, used to pin it: every token is
run through every expert (numpy fp64 matmul), experts are ranked with a full
lexicographic sort, and the chosen outputs are combined with the renormalised
softmax weights. bf16 rounding is done on the double's bit pattern (truncate,
then step up by one bf16 ulp when past the midpoint or at an odd tie), a
different method from the oracle's.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(b):
    return (np.asarray(b).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16_bits_method(v):
    """Round doubles to bf16 (nearest, ties to even) by masking mantissa bits."""
    v = np.asarray(v, dtype=np.float64)
    u = v.view(np.uint64)
    drop = np.uint64(52 - 7)  # bf16 keeps 7 explicit mantissa bits
    mask = np.uint64((1 << 45) - 1)
    trunc_u = u & ~mask
    rem = u & mask
    half = np.uint64(1 << 44)
    lsb = (trunc_u >> drop) & np.uint64(1)
    up = (rem > half) | ((rem == half) & (lsb == np.uint64(1)))
    out_u = np.where(up, trunc_u + (np.uint64(1) << drop), trunc_u)
    out = out_u.view(np.float64)
    return np.where(v == 0, v, out)


def dense_layer(x, w_router, bias, gate_up, down, k, sel="bf16"):
    """x [T,H] f64; w_router [H,E]; gate_up [E,H,2I]; down [E,I,H] (all f64).

    Returns dict(out, ids, w, logits)."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    E = w_router.shape[1]
    I = down.shape[1]
    logits = x @ np.asarray(w_router, np.float64)
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)
    if sel == "bf16":
        v = round_bf16_bits_method(logits)
    else:
        v = logits.astype(np.float32).astype(np.float64)
    p = np.exp(v - v.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ids = np.empty((T, k), np.int64)
    w = np.empty((T, k))
    eidx = np.arange(E)
    for t in range(T):
        order = np.lexsort((eidx, -v[t]))  # primary: value desc, then id asc
        ids[t] = order[:k]
        w[t] = p[t, order[:k]] / p[t, order[:k]].sum()
    # every token through every expert
    Y = np.empty((E, T, H))
    for e in range(E):
        a = x @ np.asarray(gate_up[e], np.float64)
        g, u = a[:, :I], a[:, I:]
        h = g / (1.0 + np.exp(-g)) * u
        Y[e] = h @ np.asarray(down[e], np.float64)
    out = np.zeros((T, H))
    for j in range(k):
        out += w[:, j:j + 1] * Y[ids[:, j], np.arange(T)]
    return {"out": out, "ids": ids, "w": w, "logits": logits}


def swiglu_ffn(x, gate_up, down):
    """Single dense SwiGLU FFN (the dense-MLP special case)."""
    x = np.asarray(x, np.float64)
    I = down.shape[0]
    a = x @ np.asarray(gate_up, np.float64)
    g, u = a[:, :I], a[:, I:]
    return (g / (1.0 + np.exp(-g)) * u) @ np.asarray(down, np.float64)
