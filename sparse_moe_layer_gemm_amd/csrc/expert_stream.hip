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
//    scales are applied to the fp32 accumulators in the epilogue.
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

// ------------------------------------------------------------------ bf16 weights
template <bool GATE_UP>
__global__ __launch_bounds__(256) void stream_bf16_kernel(StreamGemmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int e = blockIdx.y;
  const int tile = blockIdx.x * 4 + wave;
  const int n_tiles = GATE_UP ? a.I / 64 : (a.N + 127) / 128;
  if (tile >= n_tiles) return;
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
      for (int f = 0; f < 2; ++f) o.a[f] = load_u32x4(ar.row[f] + ks * 32 + 8 * g);
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
// E4M3 code -> bf16 bits (exact; the NaN code is never produced by an encoder).
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  const uint32_t mag = c & 0x7Fu;
  uint32_t r;
  if (mag >= 8u) {
    r = (mag << 4) + (120u << 7);  // exponent bias 7 -> 127, 3 mantissa bits on top
  } else {
    // subnormal: m * 2^-9, normalised into bf16
    r = mag == 0u ? 0u
        : mag == 1u ? (118u << 7)
        : mag <= 3u ? ((119u << 7) | ((mag & 1u) << 6))
                    : ((120u << 7) | ((mag & 3u) << 5));
  }
  return r | ((c & 0x80u) << 8);
}

// E2M1 code (4 bits) -> bf16 bits.
__device__ __forceinline__ uint32_t e2m1_to_bf16(uint32_t n) {
  const uint32_t mag = n & 7u;
  const uint32_t r = mag >= 2u ? ((((mag >> 1) + 126u) << 7) | ((mag & 1u) << 6))
                               : (mag ? 0x3F00u : 0u);
  return r | ((n & 8u) << 12);
}

// 8 consecutive E4M3 codes (two dwords) -> B fragment (4 dwords of bf16 pairs).
__device__ __forceinline__ u32x4 fp8x8_to_frag(uint32_t d0, uint32_t d1) {
  u32x4 f;
  f[0] = e4m3_to_bf16(d0 & 0xFFu) | (e4m3_to_bf16((d0 >> 8) & 0xFFu) << 16);
  f[1] = e4m3_to_bf16((d0 >> 16) & 0xFFu) | (e4m3_to_bf16(d0 >> 24) << 16);
  f[2] = e4m3_to_bf16(d1 & 0xFFu) | (e4m3_to_bf16((d1 >> 8) & 0xFFu) << 16);
  f[3] = e4m3_to_bf16((d1 >> 16) & 0xFFu) | (e4m3_to_bf16(d1 >> 24) << 16);
  return f;
}

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) scaled by an
// E4M3 block scale -> B fragment. The product has at most 6 significant bits,
// so it is exact in fp32 and its upper half is the exact bf16 value.
__device__ __forceinline__ u32x4 fp4x8_to_frag(uint32_t d, float scale) {
  u32x4 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t byte = (d >> (8 * i)) & 0xFFu;
    const float v0 = bf16_bits_to_f32(e2m1_to_bf16(byte & 0xFu)) * scale;
    const float v1 = bf16_bits_to_f32(e2m1_to_bf16(byte >> 4)) * scale;
    f[i] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);
  }
  return f;
}

// K-contiguous quantised weights. Per "super step" a lane reads 16 B of each of
// its 8 columns: FP8 -> 16 K values (2 MFMA K steps), FP4 -> 32 K values (4).
// In MFMA s of a super step the lane's K block is kb + G*g + 8s (G = 16 or 32);
// the A fragments use the same K assignment.
template <int WF, bool GATE_UP>
__global__ __launch_bounds__(256) void stream_kmajor_kernel(StreamGemmArgs a) {
  constexpr int G = (WF == W_FP8) ? 16 : 32;  // K values per lane per super step
  constexpr int NS = G / 8;                   // MFMA K steps per super step
  constexpr int SPAN = 4 * G;                 // K per super step
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int e = blockIdx.y;
  const int tile = blockIdx.x * 4 + wave;
  const int n_tiles = GATE_UP ? a.I / 64 : (a.N + 127) / 128;
  if (tile >= n_tiles) return;
  const int r0 = a.offsets[e];
  const int cnt = a.offsets[e + 1] - r0;
  if (cnt <= 0) return;
  const int K = a.K, N = a.N;

  int colv[8];
  bool cok[8];
#pragma unroll
  for (int cg = 0; cg < 8; ++cg) {
    if (GATE_UP)
      colv[cg] = cg < 4 ? tile * 64 + 16 * cg + j : a.I + tile * 64 + 16 * (cg - 4) + j;
    else
      colv[cg] = tile * 128 + 16 * cg + j;
    cok[cg] = colv[cg] < N;
  }
  const uint8_t* wq = static_cast<const uint8_t*>(a.w);
  const size_t row_bytes = (WF == W_FP8) ? (size_t)K : (size_t)K / 2;
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  const int nss = (K + SPAN - 1) / SPAN;

  for (int mc = 0; mc < cnt; mc += MROWS) {
    const int nf = (cnt - mc) > 16 ? 2 : 1;
    const ARows ar = a_rows(a, GATE_UP, r0, cnt, mc, j);
    f32x4 acc[2][8];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int ss = 0; ss < nss; ++ss) {
      const int kl = ss * SPAN + G * g;  // this lane's first K index
      const bool k_ok = kl < K;
      u32x4 braw[8];
      uint32_t sraw[8];
#pragma unroll
      for (int cg = 0; cg < 8; ++cg) {
        const bool ok = k_ok && cok[cg];
        const size_t rowoff = ((size_t)e * N + (cok[cg] ? colv[cg] : 0)) * row_bytes;
        braw[cg] = ok ? load_w(wq + rowoff + ((WF == W_FP8) ? kl : kl / 2)) : zero;
        if (WF == W_FP4) {
          const uint8_t* sp = static_cast<const uint8_t*>(a.w_scale) +
                              ((size_t)e * N + (cok[cg] ? colv[cg] : 0)) * (K / 16) + kl / 16;
          sraw[cg] = ok ? (uint32_t) * reinterpret_cast<const uint16_t*>(sp) : 0u;
        }
      }
      u32x4 af[2][NS];
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int s = 0; s < NS; ++s)
          af[f][s] = (f < nf && ar.valid[f] && k_ok) ? load_u32x4(ar.row[f] + kl + 8 * s) : zero;

#pragma unroll
      for (int cg = 0; cg < 8; ++cg) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          u32x4 bf;
          if (WF == W_FP8) {
            bf = fp8x8_to_frag(braw[cg][2 * (s & 1)], braw[cg][2 * (s & 1) + 1]);
          } else {
            const uint32_t sc = (s < 2) ? (sraw[cg] & 0xFFu) : (sraw[cg] >> 8);
            bf = fp4x8_to_frag(braw[cg][s], bf16_bits_to_f32(e4m3_to_bf16(sc)));
          }
#pragma unroll
          for (int f = 0; f < 2; ++f)
            if (f < nf) acc[f][cg] = mfma_bf16(af[f][s], bf, acc[f][cg]);
        }
      }
    }

    // epilogue: lane (g, j) holds rows 16f + 4g + r of column colv[cg]
    const float gsc = (WF == W_FP4) ? a.w_gscale[e] : 1.f;
    const float* chs = (WF == W_FP8) ? static_cast<const float*>(a.w_scale) + (size_t)e * N : nullptr;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (f >= nf) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mc + 16 * f + 4 * g + r;
        if (m >= cnt) continue;
        if (GATE_UP) {
#pragma unroll
          for (int cg = 0; cg < 4; ++cg) {
            float gv = acc[f][cg][r], uv = acc[f][cg + 4][r];
            if (WF == W_FP8) {
              gv *= chs[colv[cg]];
              uv *= chs[colv[cg + 4]];
            } else {
              gv *= gsc;
              uv *= gsc;
            }
            a.h_out[(size_t)(r0 + m) * a.I + colv[cg]] = (uint16_t)f32_to_bf16_bits(silu(gv) * uv);
          }
        } else {
#pragma unroll
          for (int cg = 0; cg < 8; ++cg)
            if (cok[cg]) {
              const float sc = (WF == W_FP8) ? chs[colv[cg]] : gsc;
              store_rows(a.y_out + (size_t)(r0 + m) * N + colv[cg], acc[f][cg][r] * sc);
            }
        }
      }
    }
  }
}

template <bool GU>
hipError_t launch_one(int wfmt, const StreamGemmArgs& a, hipStream_t st) {
  const int n_tiles = GU ? a.I / 64 : (a.N + 127) / 128;
  dim3 grid((n_tiles + 3) / 4, a.E);
  if (wfmt == W_BF16 && a.ksplit > 1) {
    grid.z = a.ksplit;
    stream_bf16_kernel<GU><<<grid, 256, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int P = (int)(a.part_stride / a.N);
    const long long items = (long long)P * (GU ? a.I : a.N) / 4;
    const unsigned blocks = (unsigned)std::min<long long>((items + 255) / 256, 4096);
    if (GU)
      stream_reduce_gu_kernel<<<blocks, 256, 0, st>>>(a.part, a.ksplit, a.part_stride, P, a.I, a.h_out);
    else
      stream_reduce_dn_kernel<<<blocks, 256, 0, st>>>(a.part, a.ksplit, a.part_stride, P, a.N, a.y_out);
    return hipGetLastError();
  }
  switch (wfmt) {
    case W_BF16: stream_bf16_kernel<GU><<<grid, 256, 0, st>>>(a); break;
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
// at least 8 K steps (256 of K) per split.
StreamSplit stream_split_plan(long long P, int E, int K, int N, bool gate_up) {
  const long long touched = std::min<long long>(E, P);
  const long long slices = gate_up ? N / 128 : (N + 127) / 128;
  const int nk = K / 32;
  const long long waves = std::max<long long>(1, touched * slices);
  long long s = (4096 + waves - 1) / waves;
  s = std::min<long long>(s, std::max(1, nk / 8));
  s = std::min<long long>(s, kMaxStreamSplit);
  if (s <= 1) return StreamSplit{1, nk};
  const int ksteps = (int)((nk + s - 1) / s);
  return StreamSplit{(nk + ksteps - 1) / ksteps, ksteps};
}

size_t stream_ws_bytes(long long P, int E, int H, int I) {
  const StreamSplit gu = stream_split_plan(P, E, H, 2 * I, true);
  const StreamSplit dn = stream_split_plan(P, E, I, H, false);
  size_t b = 0;
  if (gu.ksplit > 1) b = std::max(b, (size_t)gu.ksplit * (size_t)P * 2 * I * sizeof(float));
  if (dn.ksplit > 1) b = std::max(b, (size_t)dn.ksplit * (size_t)P * H * sizeof(float));
  return b;
}

hipError_t launch_expert_stream(int wfmt, bool gate_up, const StreamGemmArgs& a, hipStream_t st) {
  return gate_up ? launch_one<true>(wfmt, a, st) : launch_one<false>(wfmt, a, st);
}

}  // namespace moe
