"""Seeded synthetic inputs for the routed MoE layer of Beam (input generation only).

This module draws the layer's inputs: activations, router weights (with an
optional load-shaping bias) and expert weights, stored in the formats the layer
consumes (fp32, bf16, or NVFP4/FP8 codes with their scales). It holds no step
of the layer's own arithmetic (no logits, routing, permute, expert product or
finalize): the oracle and the GPU path both consume what it makes, and neither
is imported here.

The layer's shape comes from the pages: hidden 5120 (the K of the (5120, 256)
router GEMM, vLLM PR #61978 "Day-0 support for Reflection's Beam-1.0", Status
table, row #62042) and 8 of 256 routed experts per token (vLLM recipe
"reflection/Beam-1.0-501B-A23B", Guide > Overview). The expert width I=1536,
the distributions and the Zipf load are stated synthetic conventions; the
NVFP4 recipe (one E4M3 scale per 16 consecutive K elements plus one fp32 scale
per expert and matrix) is the encoding this layer's quantised variant uses for
its routed experts only (same recipe page, Guide > Variants).

Every random tensor comes from ``numpy.random.default_rng([seed, tensor, expert])``
(PCG64), so any single expert can be regenerated on its own, on any machine.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from scipy.special import ndtri

# tensor ids for the seed sequence
_T_X, _T_WR, _T_WGU, _T_WD, _T_ZIPF = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One synthetic workload of the layer."""

    name: str
    seed: int
    T: int
    H: int
    E: int
    k: int
    I: int
    x_dtype: str = "bf16"  # "f32" | "bf16"
    w_dtype: str = "bf16"  # "f32" | "bf16" | "fp8" | "fp4"
    router_only: bool = False
    zipf_s: float | None = None  # per-expert router bias shaping the load
    weight_seed: int | None = None  # expert weights drawn from this seed instead
    qmode: str = "w"  # quantised weights: "w" (exact dequant, bf16 MFMA) | "f8" (fp8 MFMA)

    @property
    def pairs(self) -> int:
        return self.T * self.k

    @property
    def logits_dtype(self) -> str:
        # the router GEMM emits bf16 logits; the all-fp32 tiny case keeps fp32
        return "f32" if self.x_dtype == "f32" else "bf16"

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


#: The five workloads: a tiny all-fp32 layer, the router alone at Beam's shape,
#: Beam decode (T=128), Beam prefill (8 x 2048 tokens, Zipf(1.1) expert load)
#: and Beam with NVFP4 experts (T=4096).
CONFIGS: dict[str, MoEConfig] = {
    "tiny_fp32": MoEConfig("tiny_fp32", 0, T=64, H=512, E=32, k=4, I=256,
                           x_dtype="f32", w_dtype="f32"),
    "router_t128": MoEConfig("router_t128", 1, T=128, H=5120, E=256, k=8, I=1536,
                             router_only=True),
    "decode_t128": MoEConfig("decode_t128", 2, T=128, H=5120, E=256, k=8, I=1536),
    "prefill_t16384_zipf": MoEConfig("prefill_t16384_zipf", 3, T=16384, H=5120, E=256,
                                     k=8, I=1536, zipf_s=1.1, weight_seed=2),
    "nvfp4_t4096": MoEConfig("nvfp4_t4096", 4, T=4096, H=5120, E=256, k=8, I=1536,
                             w_dtype="fp4"),
}


def _rng(seed: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tensor, expert])


def _normal(seed: int, tensor: int, expert: int, shape, std: float) -> np.ndarray:
    a = _rng(seed, tensor, expert).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 storage (round to nearest, ties to even) -> uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- format encoders
# Encoders only (value -> code); decoding belongs to each consumer.
# E4M3 is the OCP "fn" variant (bias 7, no infinities, 0x7F = NaN, max 448);
# E2M1 is the OCP MX FP4 element (bias 1, max 6).

def _e4m3_positive_table() -> np.ndarray:
    codes = np.arange(0x7F)  # 0..126 are the finite non-negative codes
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3_POS = _e4m3_positive_table()
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _round_to_grid(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid point to mag >= 0 (saturating), ties to the even index."""
    mag = np.minimum(mag, grid[-1])
    hi = np.clip(np.searchsorted(grid, mag, side="left"), 1, len(grid) - 1)
    lo = hi - 1
    dlo = mag - grid[lo]
    dhi = grid[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def encode_e4m3_table(v: np.ndarray) -> np.ndarray:
    """Reference encoder: nearest value of the positive E4M3 table, ties to even."""
    v = np.asarray(v, dtype=np.float64)
    idx = _round_to_grid(np.abs(v), _E4M3_POS)
    return (idx | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def encode_e2m1_table(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    idx = _round_to_grid(np.abs(v), _E2M1_POS)
    return (idx | np.where(np.signbit(v), 0x8, 0)).astype(np.uint8)


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3 codes, nearest with ties to even, saturating at 448.

    Normal range: round the fp32 mantissa to 3 bits on the bit pattern;
    below 2^-6: multiples of the subnormal quantum 2^-9 (np.rint is RNE).
    """
    v = np.asarray(v, dtype=np.float32)
    mag = np.minimum(np.abs(v), np.float32(448.0))
    u = mag.view(np.uint32)
    r = (u + np.uint32((1 << 19) - 1) + ((u >> np.uint32(20)) & np.uint32(1))) >> np.uint32(20)
    exp = (r >> np.uint32(3)).astype(np.int32) - 127 + 7
    normal = ((exp << 3) | (r & np.uint32(7)).astype(np.int32))
    sub = np.rint(mag * np.float32(512.0)).astype(np.int32)
    code = np.where(mag < np.float32(2.0 ** -6), sub, normal)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """fp32 values -> E2M1 codes, nearest with ties to even (saturating at 6).

    The grid is 0, .5, 1, 1.5, 2, 3, 4, 6; each midpoint goes to the even index.
    """
    v = np.asarray(v, dtype=np.float32)
    m = np.abs(v)
    idx = ((m > 0.25).astype(np.uint8) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5)
           + (m >= 3.5) + (m > 5.0))
    return (idx | np.where(np.signbit(v), 0x8, 0)).astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., K] 4-bit codes -> [..., K/2] bytes; element 2j in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def quantize_nvfp4(w_nk: np.ndarray):
    """NVFP4-encode one matrix stored [N, K] (K contiguous).

    Global scale s_g = amax / (448 * 6); per 16-element K block the E4M3 scale
    s_b = RNE_e4m3(amax_blk / (6 s_g)); codes q = RNE_e2m1_sat(w / (s_b s_g)).
    Returns (packed [N, K/2] u8, block scales [N, K/16] u8 (E4M3), s_g float32).
    """
    N, K = w_nk.shape
    blk = np.asarray(w_nk, dtype=np.float32).reshape(N, K // 16, 16)
    amax_b = np.max(np.abs(blk), axis=2)
    amax = float(amax_b.max())
    s_g = np.float32(amax / (448.0 * 6.0)) if amax > 0 else np.float32(1.0)
    sb_codes = encode_e4m3(amax_b / (np.float32(6.0) * s_g))
    sb_val = _E4M3_POS[sb_codes & 0x7F].astype(np.float32)
    denom = (sb_val * s_g)[:, :, None]
    safe = np.where(denom > 0, denom, np.float32(1.0))
    scaled = np.where(denom > 0, blk / safe, np.float32(0.0))
    q = encode_e2m1(scaled).reshape(N, K)
    return pack_nibbles(q), sb_codes, s_g


def quantize_fp8_channel(w_nk: np.ndarray):
    """FP8 E4M3 with one fp32 scale per output channel: s = amax_row / 448."""
    w = np.asarray(w_nk, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = encode_e4m3(w / s[:, None])
    return q, s


# ---------------------------------------------------------------- tensors
def gen_x(cfg: MoEConfig, T: int | None = None) -> np.ndarray:
    """Activations x ~ N(0,1), [T, H]: float32, or bf16 bits (uint16)."""
    T = cfg.T if T is None else T
    x = _normal(cfg.seed, _T_X, 0, (T, cfg.H), 1.0)
    return x if cfg.x_dtype == "f32" else f32_to_bf16_bits(x)


def zipf_target_load(cfg: MoEConfig) -> np.ndarray:
    """Target tokens per expert: k*T*p_rank, p_r ~ r^-s over a seeded ranking, capped at T.

    The excess of capped experts is spread over the others in proportion to
    their share (water filling) until no expert exceeds T.
    """
    E, T, k = cfg.E, cfg.T, cfg.k
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** -float(cfg.zipf_s)
    p /= p.sum()
    perm = _rng(cfg.seed, _T_ZIPF).permutation(E)
    load = np.empty(E)
    load[perm] = k * T * p
    capped = np.zeros(E, dtype=bool)
    for _ in range(E):
        over = (load > T) & ~capped
        if not over.any():
            break
        capped |= over
        load[capped] = T
        rest = k * T - T * capped.sum()
        free = ~capped
        load[free] *= rest / load[free].sum()
    return load


def zipf_bias(cfg: MoEConfig) -> np.ndarray:
    """Per-expert router bias that shapes the expert load towards Zipf(s).

    Without bias every logit is close to N(0, 1) (x ~ N(0,1), W_r ~ N(0, 1/H)).
    Treating the per-token top-k threshold as a constant, expert e is picked
    with probability Phi(b_e), so b_e = Phi^-1(load_e / T); experts whose
    target is every token get a bias far above any logit.
    """
    q = zipf_target_load(cfg) / cfg.T
    q = np.clip(q, 1e-9, 1.0)
    b = np.where(q >= 1.0, 12.0, ndtri(np.minimum(q, 1.0 - 1e-12)))
    return b.astype(np.float32)


def gen_router(cfg: MoEConfig):
    """Router weights W_r ~ N(0, 1/H), fp32 [H, E]; bias [E] fp32 or None."""
    wr = _normal(cfg.seed, _T_WR, 0, (cfg.H, cfg.E), 1.0 / np.sqrt(cfg.H))
    bias = zipf_bias(cfg) if cfg.zipf_s is not None else None
    return wr, bias


def _wseed(cfg: MoEConfig) -> int:
    return cfg.seed if cfg.weight_seed is None else cfg.weight_seed


def gen_expert_f32(cfg: MoEConfig, e: int):
    """One expert's fp32 draws: gate_up [H, 2I] ~ N(0,1/H), down [I, H] ~ N(0,1/I)."""
    s = _wseed(cfg)
    gu = _normal(s, _T_WGU, e, (cfg.H, 2 * cfg.I), 1.0 / np.sqrt(cfg.H))
    dn = _normal(s, _T_WD, e, (cfg.I, cfg.H), 1.0 / np.sqrt(cfg.I))
    return gu, dn


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gen_experts(cfg: MoEConfig, experts=None) -> dict:
    """Stacked expert weights in the config's storage format.

    f32/bf16: gate_up [E, H, 2I], down [E, I, H] (float32, or bf16 bits uint16).
    fp4: gate_up [E, 2I, H/2] u8, gate_up_scale [E, 2I, H/16] u8 (E4M3),
         gate_up_gscale [E] f32, down [E, H, I/2], down_scale [E, H, I/16], down_gscale [E].
    fp8: gate_up [E, 2I, H] u8 (E4M3), gate_up_scale [E, 2I] f32, down [E, H, I], down_scale [E, H].
    ``experts`` restricts generation to a subset (stacked in that order).
    """
    ids = list(range(cfg.E)) if experts is None else list(experts)
    n, H, I = len(ids), cfg.H, cfg.I
    dt = cfg.w_dtype
    out: dict = {"dtype": dt}
    if dt == "f32":
        out["gate_up"] = np.empty((n, H, 2 * I), np.float32)
        out["down"] = np.empty((n, I, H), np.float32)
    elif dt == "bf16":
        out["gate_up"] = np.empty((n, H, 2 * I), np.uint16)
        out["down"] = np.empty((n, I, H), np.uint16)
    elif dt == "fp4":
        out["gate_up"] = np.empty((n, 2 * I, H // 2), np.uint8)
        out["gate_up_scale"] = np.empty((n, 2 * I, H // 16), np.uint8)
        out["gate_up_gscale"] = np.empty((n,), np.float32)
        out["down"] = np.empty((n, H, I // 2), np.uint8)
        out["down_scale"] = np.empty((n, H, I // 16), np.uint8)
        out["down_gscale"] = np.empty((n,), np.float32)
    elif dt == "fp8":
        out["gate_up"] = np.empty((n, 2 * I, H), np.uint8)
        out["gate_up_scale"] = np.empty((n, 2 * I), np.float32)
        out["down"] = np.empty((n, H, I), np.uint8)
        out["down_scale"] = np.empty((n, H), np.float32)
    else:
        raise ValueError(dt)

    def one(slot: int):
        gu, dn = gen_expert_f32(cfg, ids[slot])
        if dt == "f32":
            out["gate_up"][slot] = gu
            out["down"][slot] = dn
        elif dt == "bf16":
            out["gate_up"][slot] = f32_to_bf16_bits(gu)
            out["down"][slot] = f32_to_bf16_bits(dn)
        elif dt == "fp4":
            q, sb, sg = quantize_nvfp4(np.ascontiguousarray(gu.T))
            out["gate_up"][slot], out["gate_up_scale"][slot], out["gate_up_gscale"][slot] = q, sb, sg
            q, sb, sg = quantize_nvfp4(np.ascontiguousarray(dn.T))
            out["down"][slot], out["down_scale"][slot], out["down_gscale"][slot] = q, sb, sg
        else:
            q, s = quantize_fp8_channel(np.ascontiguousarray(gu.T))
            out["gate_up"][slot], out["gate_up_scale"][slot] = q, s
            q, s = quantize_fp8_channel(np.ascontiguousarray(dn.T))
            out["down"][slot], out["down_scale"][slot] = q, s

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(n)))
    return out


def gen_layer(cfg: MoEConfig, with_experts: bool = True) -> dict:
    """All inputs of one workload as host arrays."""
    wr, bias = gen_router(cfg)
    d = {"cfg": cfg, "x": gen_x(cfg), "w_router": wr, "bias": bias}
    if with_experts and not cfg.router_only:
        d["experts"] = gen_experts(cfg)
    return d
