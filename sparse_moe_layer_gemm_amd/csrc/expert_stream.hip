// Grouped SwiGLU expert GEMMs of Beam's routed MoE layer for few rows per
// expert (decode-sized batches), on gfx950 MFMA.
//
// The pages name the pieces: per-expert GEMMs with gate and up merged into
// one projection ("merged projections", UpstreamBeat "vLLM adds day-zero
// Reflection Beam serving...", section "Agents worked on the serving path"),
// and a routed-experts-only NVFP4 variant run with BF16 activations (vLLM
// recipe "reflection/Beam-1.0-501B-A23B", Guide > Variants).
//
// At a few rows per expert the work is bound by streaming the touched
// experts' weights from HBM, so the schedule is built around reading every
// weight byte exactly once per 32 rows:
//  - a wavefront owns a 128-column slice of one expert's matrix (gate/up: 64
//    gate + 64 up columns, so SwiGLU is formed in registers) and walks the
//    whole K dimension with one K step of loads in flight ahead of the MFMAs;
//  - the A operand (gathered x rows, or h rows) is read straight from global
//    memory; it is small and stays in L2;
//  - bf16 weights are stored [K, N] (N contiguous). A lane loads 8 rows x 8
//    columns (8 x 16 B, coalesced along N) and transposes them in registers:
//    column c's 8 K values become the B fragment of MFMA c, so the 8 MFMAs of
//    a K step cover 8 columns per lane at a column stride of 1 and no LDS is
//    used at all;
//  - FP8 and NVFP4 weights are stored [N, K] (K contiguous): a lane loads 16 B
//    of one column and dequantises it exactly to bf16 in registers (E4M3 and
//    E2M1 x E4M3 products fit in bf16); per-channel and per-expert fp32
//    scales are applied to the fp32 accumulators in the epilogue;
//  - with few touched experts (small batches) there are too few slices to
//    keep HBM busy, so K is split over the grid's z dimension: the splits
//    write fp32 partial sums and a reduction kernel forms h or y, adding them
//    in split order (up to 32 pairs the down kernel forms h itself, and the
//    layer's finalize may add y's partial sums instead); and the grid has one
//    row per expert that can have rows, each row finding its expert among the
//    non-empty ones.
// MFMA v_mfma_f32_16x16x32_bf16: lane l supplies A row l%16 / B column l%16,
// K block l/16 (8 values); the result lane l holds rows 4*(l/16)+r of column
// l%16.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int MROWS = 32;  // rows per pass (two 16-row MFMA fragments)

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Weight loads: every weight byte is read once per pass, so they bypass the
// caches' retention (nontemporal); measured on gfx950 this lifts a plain
// streaming read from ~6.3 to ~7.0 TB/s.
__device__ __forceinline__ u32x4 load_w(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Rows of the A operand for one 32-row pass: pointer per fragment + validity.
struct ARows {
  const uint16_t* row[2];
  bool valid[2];
};

__device__ __forceinline__ ARows a_rows(const StreamGemmArgs& a, bool gate_up, int r0, int cnt,
                                        int mc, int j) {
  ARows ar;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int m = mc + 16 * f + j;
    ar.valid[f] = m < cnt;
    size_t row = 0;
    if (ar.valid[f]) row = gate_up ? (size_t)(a.sorted_pair[r0 + m] / a.k) : (size_t)(r0 + m);
    ar.row[f] = a.a + row * a.K;
  }
  return ar;
}

// The expert of grid row `slot`. With one row per expert (gridDim.y == E) it
// is the row itself; with fewer rows (min(E, P) < E: few pairs, so most
// experts are empty) it is the slot-th expert that has rows, found from the
// offsets by ballots (every lane of the wavefront gets the same answer), or
// -1 when fewer experts have rows.
__device__ __forceinline__ int slot_expert(const int32_t* __restrict__ offsets, int E, int slot,
                                           int lane) {
  if ((int)gridDim.y == E) return slot;
  int o0[4], o1[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {  // E <= 256: lane l looks at experts l, l+64, l+128, l+192
    const int e = 64 * c + lane;
    o0[c] = offsets[e < E ? e : 0];
    o1[c] = offsets[e < E ? e + 1 : 0];
  }
  const uint64_t below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bool nz = 64 * c + lane < E && o1[c] > o0[c];
    const uint64_t m = __ballot(nz);
    const int want = slot - base;
    if (want < __popcll(m)) {
      const uint64_t hit = __ballot(nz && __popcll(m & below) == want);
      return 64 * c + __builtin_ctzll(hit);
    }
    base += __popcll(m);
  }
  return -1;
}

// ------------------------------------------------------------------ bf16 weights
// FOLD (down only, at most 32 rows per expert): the A operand, h, is formed
// in LDS by the whole workgroup from the gate/up split partial sums before the
// K loop (h = bf16(silu(sum of gate) * sum of up), splits added in order, as
// the reduction kernel does), so the gate/up reduction needs no launch of its
// own; the workgroups of the first column group also write it to h_out. Until
// that barrier no wavefront leaves early.
template <bool GATE_UP, bool FOLD = false>
__global__ __launch_bounds__(256) void stream_bf16_kernel(StreamGemmArgs a) {
  static_assert(!(FOLD && GATE_UP), "h is folded into the down GEMM only");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int tile = blockIdx.x * 4 + wave;
  const int n_tiles = GATE_UP ? a.I / 64 : (a.N + 127) / 128;
  if constexpr (!FOLD)
    if (tile >= n_tiles) return;
  // the expert, its rows and the K range are the same for the whole workgroup
  const int e = slot_expert(a.offsets, a.E, blockIdx.y, lane);
  if (e < 0) return;
  const int r0 = a.offsets[e];
  const int cnt = a.offsets[e + 1] - r0;
  if (cnt <= 0) return;

  const int K = a.K, N = a.N;
  int col;  // first of this lane's 8 consecutive columns
  if (GATE_UP)
    col = (j < 8) ? tile * 64 + 8 * j : a.I + tile * 64 + 8 * (j - 8);
  else
    col = tile * 128 + 8 * j;
  const bool col_ok = col < N;
  const uint16_t* wb = static_cast<const uint16_t*>(a.w) + (size_t)e * K * N + (col_ok ? col : 0);
  const int nk = K / 32;
  // this wavefront's K steps (all of them unless K is split)
  const int split = blockIdx.z;
  const int ks0 = a.ksplit > 1 ? split * a.ksteps : 0;
  const int ks1 = a.ksplit > 1 ? min(nk, ks0 + a.ksteps) : nk;
  if (ks0 >= ks1) return;

  extern __shared__ __align__(16) uint8_t hl[];  // FOLD: 32 rows of h, hlds_stride bytes each
  if constexpr (FOLD) {
    const int q = (ks1 - ks0) * 8;  // float4 columns of h this split reads
    const int hc0 = ks0 * 32;
    for (int it = threadIdx.x; it < MROWS * q; it += 256) {
      const int m = it / q;
      const int c = 4 * (it - m * q);
      uint2 pk = make_uint2(0u, 0u);  // rows past the expert's end: zeros, never stored
      if (m < cnt) {
        const float* pg = a.hpart + (size_t)(r0 + m) * 2 * a.I + hc0 + c;
        f32x4 gv[kMaxStreamSplit], uv[kMaxStreamSplit];
#pragma unroll
        for (int sp = 0; sp < kMaxStreamSplit; ++sp)
          if (sp < a.hsplit) {
            gv[sp] = *reinterpret_cast<const f32x4*>(pg + sp * a.hpart_stride);
            uv[sp] = *reinterpret_cast<const f32x4*>(pg + sp * a.hpart_stride + a.I);
          }
        f32x4 gs = gv[0], us = uv[0];
#pragma unroll
        for (int sp = 1; sp < kMaxStreamSplit; ++sp)
          if (sp < a.hsplit) {
            gs += gv[sp];
            us += uv[sp];
          }
        pk.x = f32_to_bf16_bits(silu(gs[0]) * us[0]) | (f32_to_bf16_bits(silu(gs[1]) * us[1]) << 16);
        pk.y = f32_to_bf16_bits(silu(gs[2]) * us[2]) | (f32_to_bf16_bits(silu(gs[3]) * us[3]) << 16);
        // the first column group also stores the h it forms, so that h is in
        // the workspace as after the reduction kernel (the splits' K ranges
        // cover every column of h once)
        if (blockIdx.x == 0 && a.h_out)
          *reinterpret_cast<uint2*>(a.h_out + (size_t)(r0 + m) * a.I + hc0 + c) = pk;
      }
      *reinterpret_cast<uint2*>(hl + (size_t)m * a.hlds_stride + 2 * c) = pk;
    }
    __syncthreads();
    if (tile >= n_tiles) return;  // no barrier follows
  }

  for (int mc = 0; mc < cnt; mc += MROWS) {
    const int nf = (cnt - mc) > 16 ? 2 : 1;
    const ARows ar = a_rows(a, GATE_UP, r0, cnt, mc, j);
    f32x4 acc[2][8];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Every load is unconditional, from an address clamped into the matrix
    // (column 0 past N, row 0 past the expert's rows): an output element
    // depends only on its own A row and B column, and those of clamped rows
    // and columns are never stored. The A and B operands of a K step are
    // loaded together, one step ahead, into one of two register sets, so the
    // MFMAs of a step wait only for that step's loads (loads under divergent
    // branches, or a copy from one set to the other, make the compiler wait
    // for every load in flight, the next step's included).
    struct Ops {
      u32x4 a[2], b[8];
    };
    auto load = [&](int ks, Ops& o) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if constexpr (FOLD)  // row 16f + j of the LDS h rows (mc is 0: cnt <= 32)
          o.a[f] = *reinterpret_cast<const u32x4*>(hl + (size_t)(16 * f + j) * a.hlds_stride +
                                                   64 * (ks - ks0) + 16 * g);
        else
          o.a[f] = load_u32x4(ar.row[f] + ks * 32 + 8 * g);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) o.b[r] = load_w(wb + (size_t)(ks * 32 + 8 * g + r) * N);
    };
    auto step = [&](const Ops& o) {
      // 8x8 transpose: fragment for column 2q / 2q+1 from dword q of rows 2p, 2p+1
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 lo, hi;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t x0 = o.b[2 * p][q], x1 = o.b[2 * p + 1][q];
          lo[p] = (x0 & 0xFFFFu) | (x1 << 16);
          hi[p] = (x0 >> 16) | (x1 & 0xFFFF0000u);
        }
#pragma unroll
        for (int f = 0; f < 2; ++f)
          if (f < nf) {
            acc[f][2 * q] = mfma_bf16(o.a[f], lo, acc[f][2 * q]);
            acc[f][2 * q + 1] = mfma_bf16(o.a[f], hi, acc[f][2 * q + 1]);
          }
      }
    };
    Ops o0, o1;
    load(ks0, o0);
    int ks = ks0;
    for (; ks + 1 < ks1; ks += 2) {
      load(ks + 1, o1);
      step(o0);
      load(ks + 2 < ks1 ? ks + 2 : ks1 - 1, o0);  // the last pair reloads step ks1 - 1
      step(o1);
    }
    if (ks < ks1) step(o0);  // odd count: o0 holds step ks1 - 1

    if (a.ksplit > 1) {
      // fp32 partial sums of this split; lane (g, j) holds rows 16f + 4g + r
      // of columns col .. col + 7
      float* pbase = a.part + (size_t)split * a.part_stride;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (f >= nf) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mc + 16 * f + 4 * g + r;
          if (m < cnt && col_ok) {
            float* o = pbase + (size_t)(r0 + m) * N + col;
            *reinterpret_cast<f32x4*>(o) = f32x4{acc[f][0][r], acc[f][1][r], acc[f][2][r], acc[f][3][r]};
            *reinterpret_cast<f32x4*>(o + 4) =
                f32x4{acc[f][4][r], acc[f][5][r], acc[f][6][r], acc[f][7][r]};
          }
        }
      }
      continue;
    }

    // epilogue: lane (g, j) holds rows 16f + 4g + r of columns col + i (MFMA i)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (f >= nf) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mc + 16 * f + 4 * g + r;
        if (GATE_UP) {
          float hv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float v = acc[f][i][r];
            const float partner = __shfl_xor(v, 8, 64);  // up column of my gate column
            hv[i] = silu(v) * partner;
          }
          if (j < 8 && m < cnt) {
            u32x4 pk;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pk[i] = f32_to_bf16_bits(hv[2 * i]) | (f32_to_bf16_bits(hv[2 * i + 1]) << 16);
            *reinterpret_cast<u32x4*>(a.h_out + (size_t)(r0 + m) * a.I + tile * 64 + 8 * j) = pk;
          }
        } else if (m < cnt && col_ok) {
          float* o = a.y_out + (size_t)(r0 + m) * N + col;
          store_rows(o, f32x4{acc[f][0][r], acc[f][1][r], acc[f][2][r], acc[f][3][r]});
          store_rows(o + 4, f32x4{acc[f][4][r], acc[f][5][r], acc[f][6][r], acc[f][7][r]});
        }
      }
    }
  }
}

// ------------------------------------------------------------------ split-K reductions
// Sums the partial products of the splits in split order (deterministic).
// gate/up: h = bf16(silu(gate) * up) from the partial sums of both halves.
__global__ __launch_bounds__(256) void stream_reduce_gu_kernel(const float* __restrict__ part,
                                                               int S, long long sstride, int P,
                                                               int I, uint16_t* __restrict__ h) {
  const int q = I / 4;
  const long long n = (long long)P * q;
  for (long long it = (long long)blockIdx.x * 256 + threadIdx.x; it < n;
       it += (long long)gridDim.x * 256) {
    const long long r = it / q;
    const int c = (int)(it - r * q) * 4;
    const float* pg = part + r * 2 * I + c;
    f32x4 gv[kMaxStreamSplit], uv[kMaxStreamSplit];  // all loads in flight at once
#pragma unroll
    for (int sp = 0; sp < kMaxStreamSplit; ++sp)
      if (sp < S) {
        gv[sp] = *reinterpret_cast<const f32x4*>(pg + sp * sstride);
        uv[sp] = *reinterpret_cast<const f32x4*>(pg + sp * sstride + I);
      }
    f32x4 gs = gv[0], us = uv[0];
#pragma unroll
    for (int sp = 1; sp < kMaxStreamSplit; ++sp)
      if (sp < S) {
        gs += gv[sp];
        us += uv[sp];
      }
    uint2 pk;
    pk.x = f32_to_bf16_bits(silu(gs[0]) * us[0]) | (f32_to_bf16_bits(silu(gs[1]) * us[1]) << 16);
    pk.y = f32_to_bf16_bits(silu(gs[2]) * us[2]) | (f32_to_bf16_bits(silu(gs[3]) * us[3]) << 16);
    *reinterpret_cast<uint2*>(h + r * I + c) = pk;
  }
}
// down: y = sum of the partial rows.
__global__ __launch_bounds__(256) void stream_reduce_dn_kernel(const float* __restrict__ part,
                                                               int S, long long sstride, int P,
                                                               int N, float* __restrict__ y) {
  const int q = N / 4;
  const long long n = (long long)P * q;
  for (long long it = (long long)blockIdx.x * 256 + threadIdx.x; it < n;
       it += (long long)gridDim.x * 256) {
    const long long r = it / q;
    const int c = (int)(it - r * q) * 4;
    const float* pp = part + r * N + c;
    f32x4 pv[kMaxStreamSplit];
#pragma unroll
    for (int sp = 0; sp < kMaxStreamSplit; ++sp)
      if (sp < S) pv[sp] = *reinterpret_cast<const f32x4*>(pp + sp * sstride);
    f32x4 v = pv[0];
#pragma unroll
    for (int sp = 1; sp < kMaxStreamSplit; ++sp)
      if (sp < S) v += pv[sp];
    store_rows(y + r * N + c, v);
  }
}

// ------------------------------------------------------------------ FP8 / NVFP4 weights
// K-contiguous quantised weights ([E, N, K] E4M3 codes, or [E, N, K/2] E2M1
// codes with one E4M3 scale per 16 K values). Per "super step" the four lane
// groups of a column each read 32 B of it, together one whole 128 B line
// (E4M3: 32 K values per lane, E2M1: 64), plus, for E2M1, the dword of this
// lane's four block scales, with the matching A fragments; like the bf16
// kernel, a super step's loads are issued one step ahead into one of two
// register sets, unconditionally from clamped addresses. Each code line is
// consumed by the load that fetches it, so code loads skip cache retention
// (nontemporal), leaving L2 to the scale lines, which serve 8 super steps.
// (Reading half a line per super step measured 2.8x the algorithmic bytes
// fetched at decode: lines were evicted before their second half was used.)
// A wavefront owns 64 columns (gate/up: 32 gate + the 32 matching up). Codes
// become bf16 with the hardware converters (E4M3 exactly; E2M1 with the power
// of two of its block scale, then an fp32 multiply by the scale's mantissa
// factor, exact as well). Per-channel (E4M3) and per-expert (E2M1) fp32
// scales multiply the accumulators. In MFMA s of a super step lane group g
// covers K ss*SPAN + G*g + 8s .. +8, for A and B alike.
template <int WF>
struct KmShape {
  static constexpr int G = (WF == W_FP8) ? 32 : 64;  // K values per lane per super step
  static constexpr int NS = G / 8;                   // MFMA K steps per super step
  static constexpr int SPAN = 4 * G;                 // K per super step
  static constexpr int NV = 2;                       // 16 B code loads per lane and column
  static constexpr int CG = 4;                       // 16-column groups per wavefront
  static constexpr int COLS = 16 * CG;               // columns per wavefront
  // row fragments per pass: one for E2M1 (its A fragments per fragment row
  // and super step would otherwise cost a wave per SIMD of occupancy)
  static constexpr int NF = (WF == W_FP4) ? 1 : 2;
};

template <int WF, bool GATE_UP>
__global__ __launch_bounds__(256, 2) void stream_kmajor_kernel(StreamGemmArgs a) {
  using S = KmShape<WF>;
  constexpr int G = S::G, NS = S::NS, SPAN = S::SPAN, NV = S::NV, CG = S::CG, NF = S::NF;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int tile = blockIdx.x * 4 + wave;
  const int n_tiles = GATE_UP ? a.I / (S::COLS / 2) : (a.N + S::COLS - 1) / S::COLS;
  if (tile >= n_tiles) return;
  const int e = slot_expert(a.offsets, a.E, blockIdx.y, lane);
  if (e < 0) return;
  const int r0 = a.offsets[e];
  const int cnt = a.offsets[e + 1] - r0;
  if (cnt <= 0) return;
  const int K = a.K, N = a.N;
  const int nss = (K + SPAN - 1) / SPAN;
  const int split = blockIdx.z;
  const int ss0 = a.ksplit > 1 ? split * a.ksteps : 0;
  const int ss1 = a.ksplit > 1 ? min(nss, ss0 + a.ksteps) : nss;
  if (ss0 >= ss1) return;

  // this lane's CG columns (gate/up: CG/2 gate, then the matching up columns);
  // columns past N read column 0 and are never stored
  const int row_bytes = (WF == W_FP8) ? K : K / 2;
  const uint8_t* wexp = static_cast<const uint8_t*>(a.w) + (size_t)e * N * row_bytes;
  const uint8_t* sexp =
      (WF == W_FP4) ? static_cast<const uint8_t*>(a.w_scale) + (size_t)e * N * (K / 16) : nullptr;
  int colv[CG];
  bool cok[CG];
  uint32_t coff[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    constexpr int H2 = CG / 2, HC = S::COLS / 2;
    if (GATE_UP)
      colv[cg] = cg < H2 ? tile * HC + 16 * cg + j : a.I + tile * HC + 16 * (cg - H2) + j;
    else
      colv[cg] = tile * S::COLS + 16 * cg + j;
    cok[cg] = colv[cg] < N;
    coff[cg] = (uint32_t)(cok[cg] ? colv[cg] : 0);
  }
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};

  for (int mc = 0; mc < cnt; mc += 16 * NF) {
    const int nf = (NF == 2 && (cnt - mc) > 16) ? 2 : 1;
    const ARows ar = a_rows(a, GATE_UP, r0, cnt, mc, j);
    f32x4 acc[NF][CG];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < CG; ++i) acc[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct Ops {
      u32x4 a[NF][NS], b[CG][NV];
      uint32_t sc[CG];
      bool kok;  // this lane's K range lies inside K (false only in a K tail)
    };
    auto load = [&](int ss, Ops& o) {
      const int kl = ss * SPAN + G * g;
      o.kok = kl < K;
      const int kc = o.kok ? kl : 0;
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int q = 0; q < NS; ++q) o.a[f][q] = load_u32x4(ar.row[f] + kc + 8 * q);
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
#pragma unroll
        for (int v = 0; v < NV; ++v)
          o.b[cg][v] = load_w(wexp + (size_t)coff[cg] * row_bytes + (WF == W_FP8 ? kc : kc / 2) + 16 * v);
      if constexpr (WF == W_FP4) {
#pragma unroll
        for (int cg = 0; cg < CG; ++cg)  // the four block scales of this lane's 64 K values
          o.sc[cg] = *reinterpret_cast<const uint32_t*>(sexp + (size_t)coff[cg] * (K / 16) + kc / 16);
      }
    };
    auto step = [&](const Ops& o) {
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        float p2[4], fm[4];
        if constexpr (WF == W_FP4) {
#pragma unroll
          for (int b = 0; b < 4; ++b) e4m3_split((o.sc[cg] >> (8 * b)) & 0xFFu, p2[b], fm[b]);
        }
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          u32x4 bf;
          if constexpr (WF == W_FP8)
            bf = fp8_frag(o.b[cg][q >> 1][2 * (q & 1)], o.b[cg][q >> 1][2 * (q & 1) + 1]);
          else
            bf = fp4_frag(o.b[cg][q >> 2][q & 3], p2[q >> 1], fm[q >> 1]);
#pragma unroll
          for (int f = 0; f < NF; ++f)
            if (f < nf) acc[f][cg] = mfma_bf16(o.kok ? o.a[f][q] : zero, bf, acc[f][cg]);
        }
      }
    };
    // (the scheduling barriers keep each step's loads ahead of the previous
    // step's conversions, which register pressure would otherwise sink them past)
    Ops o0, o1;
    load(ss0, o0);
    int ss = ss0;
    for (; ss + 1 < ss1; ss += 2) {
      load(ss + 1, o1);
      __builtin_amdgcn_sched_barrier(0);
      step(o0);
      load(ss + 2 < ss1 ? ss + 2 : ss1 - 1, o0);  // the last pair reloads step ss1 - 1
      __builtin_amdgcn_sched_barrier(0);
      step(o1);
    }
    if (ss < ss1) step(o0);

    // epilogue: lane (g, j) holds rows 16f + 4g + r of column colv[cg]
    const float gsc = (WF == W_FP4) ? a.w_gscale[e] : 1.f;
    const float* chs = (WF == W_FP8) ? static_cast<const float*>(a.w_scale) + (size_t)e * N : nullptr;
    float csc[CG];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) csc[cg] = (WF == W_FP8) ? chs[coff[cg]] : gsc;
    float* pbase = a.ksplit > 1 ? a.part + (size_t)split * a.part_stride : nullptr;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f >= nf) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mc + 16 * f + 4 * g + r;
        if (m >= cnt) continue;
        if (pbase) {  // split K: scaled fp32 partial sums
#pragma unroll
          for (int cg = 0; cg < CG; ++cg)
            if (cok[cg]) pbase[(size_t)(r0 + m) * N + colv[cg]] = acc[f][cg][r] * csc[cg];
        } else if (GATE_UP) {
#pragma unroll
          for (int cg = 0; cg < CG / 2; ++cg) {
            const float gv = acc[f][cg][r] * csc[cg], uv = acc[f][cg + CG / 2][r] * csc[cg + CG / 2];
            a.h_out[(size_t)(r0 + m) * a.I + colv[cg]] = (uint16_t)f32_to_bf16_bits(silu(gv) * uv);
          }
        } else {
#pragma unroll
          for (int cg = 0; cg < CG; ++cg)
            if (cok[cg]) store_rows(a.y_out + (size_t)(r0 + m) * N + colv[cg], acc[f][cg][r] * csc[cg]);
        }
      }
    }
  }
}

// Columns per wavefront of the streaming kernels.
int stream_cols(int wfmt) { return wfmt == W_BF16 ? 128 : KmShape<W_FP8>::COLS; }

template <bool GU>
hipError_t launch_one(int wfmt, const StreamGemmArgs& a, hipStream_t st) {
  const int cols = stream_cols(wfmt);
  const int n_tiles = GU ? a.I / (cols / 2) : (a.N + cols - 1) / cols;
  // one grid row per expert that can have rows: at most min(E, P) do
  dim3 grid((n_tiles + 3) / 4, a.rows > 0 ? std::min(a.E, a.rows) : a.E);
  const bool fold = !GU && a.hpart != nullptr;
  if (fold && (wfmt != W_BF16 || a.rows > MROWS || a.hsplit < 1 || a.hsplit > kMaxStreamSplit ||
               MROWS * a.hlds_stride > 65536))
    return hipErrorInvalidValue;
  if (a.ksplit > 1) {
    grid.z = a.ksplit;
    switch (wfmt) {
      case W_BF16:
        if (fold)
          stream_bf16_kernel<false, true><<<grid, 256, MROWS * a.hlds_stride, st>>>(a);
        else
          stream_bf16_kernel<GU><<<grid, 256, 0, st>>>(a);
        break;
      case W_FP8: stream_kmajor_kernel<W_FP8, GU><<<grid, 256, 0, st>>>(a); break;
      case W_FP4: stream_kmajor_kernel<W_FP4, GU><<<grid, 256, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.keep_partials) return err;
    const int P = a.rows;
    const long long items = (long long)P * (GU ? a.I : a.N) / 4;
    const unsigned blocks = (unsigned)std::min<long long>((items + 255) / 256, 4096);
    if (GU)
      stream_reduce_gu_kernel<<<blocks, 256, 0, st>>>(a.part, a.ksplit, a.part_stride, P, a.I, a.h_out);
    else
      stream_reduce_dn_kernel<<<blocks, 256, 0, st>>>(a.part, a.ksplit, a.part_stride, P, a.N, a.y_out);
    return hipGetLastError();
  }
  switch (wfmt) {
    case W_BF16:
      if (fold)
        stream_bf16_kernel<false, true><<<grid, 256, MROWS * a.hlds_stride, st>>>(a);
      else
        stream_bf16_kernel<GU><<<grid, 256, 0, st>>>(a);
      break;
    case W_FP8: stream_kmajor_kernel<W_FP8, GU><<<grid, 256, 0, st>>>(a); break;
    case W_FP4: stream_kmajor_kernel<W_FP4, GU><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Wavefronts of one split: touched experts (at most min(E, P)) x column
// slices. Splits are added until about 4096 wavefronts stream (two rounds at
// two per SIMD; measured at T = 1 ... 8 this beats one exact round), keeping
// at least 8 K steps per split. A K step is 32 K values for bf16 weights and
// one super step (128 or 256 K values) for FP8 / NVFP4 weights.
StreamSplit stream_split_plan(long long P, int E, int K, int N, bool gate_up, int wfmt) {
  const int step = stream_k_step(wfmt), cols = stream_cols(wfmt);
  const long long touched = std::min<long long>(E, P);
  const long long slices = gate_up ? N / cols : (N + cols - 1) / cols;
  const int nk = (K + step - 1) / step;
  const long long waves = std::max<long long>(1, touched * slices);
  long long s = (4096 + waves - 1) / waves;
  s = std::min<long long>(s, std::max(1, nk / 8));
  s = std::min<long long>(s, kMaxStreamSplit);
  if (s <= 1) return StreamSplit{1, nk};
  const int ksteps = (int)((nk + s - 1) / s);
  return StreamSplit{(nk + ksteps - 1) / ksteps, ksteps};
}

int stream_k_step(int wfmt) {
  return wfmt == W_FP4 ? KmShape<W_FP4>::SPAN : wfmt == W_FP8 ? KmShape<W_FP8>::SPAN : 32;
}

bool stream_fold_h(long long P, int E, int H, int I, int wfmt, int* kr) {
  if (wfmt != W_BF16 || P > MROWS) return false;
  const StreamSplit gu = stream_split_plan(P, E, H, 2 * I, true, W_BF16);
  if (gu.ksplit <= 1) return false;
  const int k = stream_split_plan(P, E, I, H, false, W_BF16).ksteps * 32;
  if (MROWS * (2 * k + 16) > 65536) return false;
  *kr = k;
  return true;
}

size_t stream_gu_part_bytes(long long P, int E, int H, int I, int wfmt) {
  const StreamSplit gu = stream_split_plan(P, E, H, 2 * I, true, wfmt);
  const size_t b = gu.ksplit > 1 ? (size_t)gu.ksplit * (size_t)P * 2 * I * sizeof(float) : 0;
  return (b + 255) / 256 * 256;
}

size_t stream_ws_bytes(long long P, int E, int H, int I, int wfmt) {
  const StreamSplit gu = stream_split_plan(P, E, H, 2 * I, true, wfmt);
  const StreamSplit dn = stream_split_plan(P, E, I, H, false, wfmt);
  size_t b = 0;
  if (gu.ksplit > 1) b = std::max(b, (size_t)gu.ksplit * (size_t)P * 2 * I * sizeof(float));
  const size_t bd = dn.ksplit > 1 ? (size_t)dn.ksplit * (size_t)P * H * sizeof(float) : 0;
  int kr;
  if (stream_fold_h(P, E, H, I, wfmt, &kr))  // gate/up partials live on while down writes its own
    return stream_gu_part_bytes(P, E, H, I, wfmt) + bd;
  return std::max(b, bd);
}

hipError_t launch_expert_stream(int wfmt, bool gate_up, const StreamGemmArgs& a, hipStream_t st) {
  return gate_up ? launch_one<true>(wfmt, a, st) : launch_one<false>(wfmt, a, st);
}

}  // namespace moe
