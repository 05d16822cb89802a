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
//  - FP8 and NVFP4 weights are stored [N, K] (K contiguous); their kernels
//    (expert_stream_q.hip) run on the same grid and split-K partial sums;
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

#include "stream_common.h"

namespace moe {
namespace {

constexpr int MROWS = 32;  // rows per pass (two 16-row MFMA fragments)

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Weight loads: every weight byte is read once per pass, so they bypass the
// caches' retention (nontemporal); measured on gfx950 this lifts a plain
// streaming read from ~6.3 to ~7.0 TB/s.
#ifndef MOE_BF16_NT
#define MOE_BF16_NT 1
#endif
__device__ __forceinline__ u32x4 load_w(const void* p) {
  if constexpr (MOE_BF16_NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
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
// FOLD (down only, at most 32 rows per expert): the A operand, h, is formed
// in LDS by the whole workgroup from the gate/up split partial sums before the
// K loop (h = bf16(silu(sum of gate) * sum of up), splits added in order, as
// the reduction kernel does), so the gate/up reduction needs no launch of its
// own; the workgroups of the first column group also write it to h_out. Until
// that barrier no wavefront leaves early.
template <bool GATE_UP, bool FOLD, int NS = kMaxStreamSplit>
__device__ __forceinline__ void stream_bf16_body(const StreamGemmArgs& a) {
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

  // A and B operands of one K step, in registers
  struct Ops {
    u32x4 a[2], b[8];
  };
  auto load_b = [&](int ks, Ops& o) {
#pragma unroll
    for (int r = 0; r < 8; ++r) o.b[r] = load_w(wb + (size_t)(ks * 32 + 8 * g + r) * N);
  };
  Ops first;  // FOLD: the first step's weights, loaded while h is formed
  extern __shared__ __align__(16) uint8_t hl[];  // FOLD: 32 rows of h, hlds_stride bytes each
  if constexpr (FOLD) {
    // one h column per thread and item; the split sums of an item are loaded
    // together, unconditionally (an item past the expert's rows reads its
    // first row and is stored as zeros)
    const int q = (ks1 - ks0) * 32;  // columns of h this split reads
    const int hc0 = ks0 * 32;
    auto fold = [&](int it, bool with_b) {
      const int m = it / q;
      const int c = it - m * q;
      const bool ok = m < cnt;
      const float* pg = a.hpart + (size_t)(r0 + (ok ? m : 0)) * 2 * a.I + hc0 + c;
      // all NS split slots are loaded (slots past the split count re-read
      // split 0) so that no branch separates these loads from the weight
      // loads below; the unused slots add -0, which changes no sum
      float gv[NS], uv[NS];
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) {
        const size_t o = (size_t)(sp < a.hsplit ? sp : 0) * a.hpart_stride;
        gv[sp] = pg[o];
        uv[sp] = pg[o + a.I];
      }
      // the first item's loads are followed by the first step's weight
      // loads, which do not depend on h: the sums below wait only for the
      // older partial-sum loads, and the weights arrive meanwhile
      if (with_b) {
        __builtin_amdgcn_sched_barrier(0);
        load_b(ks0, first);
        __builtin_amdgcn_sched_barrier(0);
      }
      float gs = gv[0], us = uv[0];
#pragma unroll
      for (int sp = 1; sp < NS; ++sp) {
        gs += sp < a.hsplit ? gv[sp] : -0.0f;
        us += sp < a.hsplit ? uv[sp] : -0.0f;
      }
      const uint16_t hv = ok ? (uint16_t)f32_to_bf16_bits(silu(gs) * us) : (uint16_t)0;
      // the first column group also stores the h it forms, so that h is in
      // the workspace as after the reduction kernel (the splits' K ranges
      // cover every column of h once)
      if (ok && blockIdx.x == 0 && a.h_out) a.h_out[(size_t)(r0 + m) * a.I + hc0 + c] = hv;
      *reinterpret_cast<uint16_t*>(hl + (size_t)m * a.hlds_stride + 2 * c) = hv;
    };
    // every thread has an item below 256 (q >= 32, so they lie in the LDS rows)
    fold(threadIdx.x, true);
    for (int it = threadIdx.x + 256; it < cnt * q; it += 256) fold(it, false);
    // rows past the expert's end feed only accumulators that are never stored
    const int z0 = cnt * q > 256 ? cnt * q : 256;  // items below 256 were written above
    for (int it = z0 + threadIdx.x; it < MROWS * q; it += 256) {
      const int m = it / q;
      *reinterpret_cast<uint16_t*>(hl + (size_t)m * a.hlds_stride + 2 * (it - m * q)) = 0;
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
    auto load_a = [&](int ks, Ops& o) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if constexpr (FOLD)  // row 16f + j of the LDS h rows (mc is 0: cnt <= 32)
          o.a[f] = *reinterpret_cast<const u32x4*>(hl + (size_t)(16 * f + j) * a.hlds_stride +
                                                   64 * (ks - ks0) + 16 * g);
        else
          o.a[f] = load_u32x4(ar.row[f] + ks * 32 + 8 * g);
      }
    };
    auto load = [&](int ks, Ops& o) {
      load_a(ks, o);
      load_b(ks, o);
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
    if constexpr (FOLD) {  // the first step's weights are already in flight
      o0 = first;
      load_a(ks0, o0);
    } else {
      load(ks0, o0);
    }
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

template <bool GATE_UP>
__global__ __launch_bounds__(256) void stream_bf16_kernel(StreamGemmArgs a) {
  stream_bf16_body<GATE_UP, false>(a);
}
// down GEMM with h folded in from up to NS gate/up splits: held to two
// wavefronts per SIMD (256 registers), so that the whole small-batch grid is
// resident at once
template <int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void stream_bf16_fold_kernel(
    StreamGemmArgs a) {
  stream_bf16_body<false, true, NS>(a);
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

// Columns per wavefront of the streaming kernels.
int stream_cols(int wfmt) { return wfmt == W_BF16 ? 128 : stream_q_cols(wfmt); }

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
        if (!fold)
          stream_bf16_kernel<GU><<<grid, 256, 0, st>>>(a);
        else if (a.hsplit <= 8)
          stream_bf16_fold_kernel<8><<<grid, 256, MROWS * a.hlds_stride, st>>>(a);
        else
          stream_bf16_fold_kernel<kMaxStreamSplit><<<grid, 256, MROWS * a.hlds_stride, st>>>(a);
        break;
      default: {
        const hipError_t e = launch_stream_q(wfmt, GU, grid, a, st);
        if (e != hipSuccess) return e;
      }
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
      if (!fold)
        stream_bf16_kernel<GU><<<grid, 256, 0, st>>>(a);
      else if (a.hsplit <= 8)
        stream_bf16_fold_kernel<8><<<grid, 256, MROWS * a.hlds_stride, st>>>(a);
      else
        stream_bf16_fold_kernel<kMaxStreamSplit><<<grid, 256, MROWS * a.hlds_stride, st>>>(a);
      break;
    default: return launch_stream_q(wfmt, GU, grid, a, st);
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
  // NVFP4 weights, K already split: splits of at most 8 super steps (one
  // scale block), with which the kernel keeps a split's A rows and scales in
  // LDS for the whole pass (measured at T = 1: gate/up 3 splits of 7 instead
  // of 2 of 10, expert stage 40.1 -> 38.8 us; at T = 128, which needs no
  // split, forcing 3 splits was 5% slower)
  if (wfmt == W_FP4 && s > 1 && nk > 8) s = std::max<long long>(s, (nk + 7) / 8);
  if (s <= 1) return StreamSplit{1, nk};
  const int ksteps = (int)((nk + s - 1) / s);
  return StreamSplit{(nk + ksteps - 1) / ksteps, ksteps};
}

int stream_k_step(int wfmt) { return wfmt == W_BF16 ? 32 : stream_q_k_step(wfmt); }

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

bool stream_buffers_fit(long long P, int H, int I) {
  const long long K = H > I ? H : I;
  return P > 0 && P * K * 2 <= 0x7FFFFFFFLL && 2LL * H * I <= 0x7FFFFFFFLL;
}

hipError_t launch_expert_stream(int wfmt, bool gate_up, const StreamGemmArgs& a, hipStream_t st) {
  // the FP8 / NVFP4 kernels address A (P rows at most) and one expert's
  // weights as buffers
  if (wfmt != W_BF16 && (a.rows <= 0 || (long long)a.rows * a.K * 2 > 0x7FFFFFFFLL ||
                         (long long)a.N * a.K > 0x7FFFFFFFLL))
    return hipErrorInvalidValue;
  return gate_up ? launch_one<true>(wfmt, a, st) : launch_one<false>(wfmt, a, st);
}

}  // namespace moe
