// MoE finalize on gfx950: the weighted un-permute that closes Beam's routed
// MoE layer (vLLM PR #61978, Status table row #62366 and Remaining work name
// it as its own kernel). out[t] = sum_j w[t, j] * y_sorted[pair_pos[t*k + j]],
// fp32 accumulation in slot order, then round-to-nearest-even to bf16.
//
// Bound by HBM: every fp32 expert row is read once and every output row
// written once. One workgroup per (token, 1024-column chunk) work item, so
// that small batches still spread over the chip; the k row positions and weights are
// wave-uniform (scalar loads), each lane issues its k float4 loads together
// (rows past k repeat the first and are not added) and sums in slot order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int FCOLS = 1024;  // columns per workgroup (256 lanes x float4)

// Row positions and weights of token t's k slots (wave-uniform). Slots 8 > j >= k
// and pairs the permute left without a row (position -1: an expert id outside
// [0, E)) are not added; their loads read row 0, which always exists.
__device__ __forceinline__ void slot_rows(const int32_t* __restrict__ pair_pos,
                                          const float* __restrict__ w, long long t, int k,
                                          int (&pos)[8], float (&wt)[8], bool (&use)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = pair_pos[t * k + (j < k ? j : 0)];
    use[j] = j < k && p >= 0;
    pos[j] = use[j] ? p : 0;
    wt[j] = use[j] ? w[t * k + j] : 0.f;
  }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ y,
                                                       const int32_t* __restrict__ pair_pos,
                                                       const float* __restrict__ w, int k, int H,
                                                       int n_chunks, long long n_items,
                                                       void* __restrict__ out,
                                                       float* __restrict__ out_f32) {
  for (long long item = blockIdx.x; item < n_items; item += gridDim.x) {
    const long long t = item / n_chunks;
    const int c = (int)(item - t * n_chunks) * FCOLS + threadIdx.x * 4;
    int pos[8];
    float wt[8];
    bool use[8];
    slot_rows(pair_pos, w, t, k, pos, wt, use);
    if (c >= H) continue;
    f32x4 v[8];  // each expert row is read once: nontemporal
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (size_t)pos[j] * H + c));
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (use[j]) {
        acc.x = fmaf(wt[j], v[j].x, acc.x);
        acc.y = fmaf(wt[j], v[j].y, acc.y);
        acc.z = fmaf(wt[j], v[j].z, acc.z);
        acc.w = fmaf(wt[j], v[j].w, acc.w);
      }
    }
    if (out_f32) *reinterpret_cast<float4*>(out_f32 + (size_t)t * H + c) = acc;
    if constexpr (BF16_OUT) {
      uint2 pk;
      pk.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
      pk.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * H + c) = pk;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)t * H + c) = acc;
    }
  }
}

// The same over compact rows: fp16 values with one power-of-two scale byte
// per row and 64-column block; each value is decoded exactly to fp32
// (fp16 -> fp32, times 2^(b - 127)) and summed as above.
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void finalize_rows16_kernel(
    const uint16_t* __restrict__ y16, const uint8_t* __restrict__ ysc,
    const int32_t* __restrict__ pair_pos, const float* __restrict__ w, int k, int H, int n_chunks,
    long long n_items, void* __restrict__ out, float* __restrict__ out_f32) {
  const int nb = H / 64;
  for (long long item = blockIdx.x; item < n_items; item += gridDim.x) {
    const long long t = item / n_chunks;
    const int c = (int)(item - t * n_chunks) * FCOLS + threadIdx.x * 4;
    int pos[8];
    float wt[8];
    bool use[8];
    slot_rows(pair_pos, w, t, k, pos, wt, use);
    if (c >= H) continue;
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    u32x2v v[8];
    uint32_t sb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(y16 + (size_t)pos[j] * H + c));
      sb[j] = ysc[(size_t)pos[j] * nb + (c >> 6)];
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (use[j]) {
        const int e = (int)sb[j] - 127;
        acc.x = fmaf(wt[j], __builtin_ldexpf(f16_bits_to_f32(v[j].x & 0xffffu), e), acc.x);
        acc.y = fmaf(wt[j], __builtin_ldexpf(f16_bits_to_f32(v[j].x >> 16), e), acc.y);
        acc.z = fmaf(wt[j], __builtin_ldexpf(f16_bits_to_f32(v[j].y & 0xffffu), e), acc.z);
        acc.w = fmaf(wt[j], __builtin_ldexpf(f16_bits_to_f32(v[j].y >> 16), e), acc.w);
      }
    }
    if (out_f32) *reinterpret_cast<float4*>(out_f32 + (size_t)t * H + c) = acc;
    if constexpr (BF16_OUT) {
      uint2 pk;
      pk.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
      pk.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * H + c) = pk;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)t * H + c) = acc;
    }
  }
}

// The same from the fp32 partial sums of a split-K down GEMM, which the
// streaming kernels leave at small batches: an expert row is the sum of its S
// partial rows in split order (exactly as the split reduction forms it), then
// the k rows are added with their weights in slot order as above. Work item:
// (token, 256-column chunk); wavefront q forms the rows of slots q and q + 4
// for the chunk's 64 float4 columns (all 2 S loads issued together) and puts
// them in LDS, then wavefront 0 adds them. Folding the reduction in here saves
// a launch and a pass over the rows when the layer is latency-bound.
// NS (4, 8 or 16) bounds S: the NS loads per slot are unconditional, splits
// past S re-reading split S - 1 (not added). Loads behind a branch each would
// leave the count of loads in flight unknown, and the wait for the second
// slot's row position would then wait for the first slot's rows too.
template <bool BF16_OUT, int NS>
__global__ __launch_bounds__(256) void finalize_split_kernel(
    const float* __restrict__ part, int S, long long sstride, const int32_t* __restrict__ pair_pos,
    const float* __restrict__ w, int k, int H, int n_chunks, long long n_items,
    void* __restrict__ out, float* __restrict__ out_f32) {
  __shared__ f32x4 rows[8][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (long long item = blockIdx.x; item < n_items; item += gridDim.x) {
    const long long t = item / n_chunks;
    const int c = (int)(item - t * n_chunks) * 256 + lane * 4;
    const bool col_ok = c < H;
    bool use[2];
    const float* src[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // slot wave + 4h; unused ones read row 0, column 0
      const int j = wave + 4 * h;
      const int p = pair_pos[t * k + (j < k ? j : 0)];
      use[h] = j < k && col_ok;
      src[h] = part + (size_t)(p >= 0 ? p : 0) * H + (col_ok ? c : 0);
      if (p < 0) use[h] = false;  // no row: the slot reads as zeros below
    }
    // the token's weights go out before the partial sums: no load after the barrier
    float wt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wt[j] = j < k ? w[t * k + j] : 0.f;
    f32x4 pv[2][NS];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int sp = 0; sp < NS; ++sp)
        pv[h][sp] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(src[h] + (sp < S ? sp : S - 1) * sstride));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 v = pv[h][0];
#pragma unroll
      for (int sp = 1; sp < NS; ++sp)
        if (sp < S) v += pv[h][sp];
      if (use[h]) rows[wave + 4 * h][lane] = v;
      else if (wave + 4 * h < k && col_ok) rows[wave + 4 * h][lane] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    if (wave == 0 && col_ok) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < k) {
          const f32x4 v = rows[j][lane];
          acc.x = fmaf(wt[j], v.x, acc.x);
          acc.y = fmaf(wt[j], v.y, acc.y);
          acc.z = fmaf(wt[j], v.z, acc.z);
          acc.w = fmaf(wt[j], v.w, acc.w);
        }
      }
      if (out_f32) *reinterpret_cast<float4*>(out_f32 + (size_t)t * H + c) = acc;
      if constexpr (BF16_OUT) {
        uint2 pk;
        pk.x = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
        pk.y = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * H + c) = pk;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)t * H + c) = acc;
      }
    }
    __syncthreads();  // rows[] is rewritten by the next item
  }
}

}  // namespace

hipError_t launch_finalize_split(const float* part, int S, long long sstride,
                                 const int32_t* pair_pos, const float* w, int T, int k, int H,
                                 bool out_bf16, void* out, float* out_f32, hipStream_t st) {
  if (S < 1 || S > kMaxStreamSplit || k < 1 || k > 8) return hipErrorInvalidValue;
  const int n_chunks = (H + 255) / 256;
  const long long items = (long long)T * n_chunks;
  const unsigned grid = (unsigned)(items < (1 << 20) ? items : (1 << 20));
  auto go = [&](auto ns) {
    constexpr int NS = decltype(ns)::value;
    if (out_bf16)
      finalize_split_kernel<true, NS><<<grid, 256, 0, st>>>(part, S, sstride, pair_pos, w, k, H,
                                                            n_chunks, items, out, out_f32);
    else
      finalize_split_kernel<false, NS><<<grid, 256, 0, st>>>(part, S, sstride, pair_pos, w, k, H,
                                                             n_chunks, items, out, out_f32);
  };
  static_assert(kMaxStreamSplit == 16, "split bound buckets");
  if (S <= 4)
    go(std::integral_constant<int, 4>{});
  else if (S <= 8)
    go(std::integral_constant<int, 8>{});
  else
    go(std::integral_constant<int, 16>{});
  return hipGetLastError();
}

hipError_t launch_finalize_rows16(const uint16_t* y16, const uint8_t* y16_scale,
                                  const int32_t* pair_pos, const float* w, int T, int k, int H,
                                  bool out_bf16, void* out, float* out_f32, hipStream_t st) {
  const int n_chunks = (H + FCOLS - 1) / FCOLS;
  const long long items = (long long)T * n_chunks;
  const unsigned grid = (unsigned)(items < (1 << 20) ? items : (1 << 20));
  if (out_bf16)
    finalize_rows16_kernel<true><<<grid, 256, 0, st>>>(y16, y16_scale, pair_pos, w, k, H, n_chunks,
                                                       items, out, out_f32);
  else
    finalize_rows16_kernel<false><<<grid, 256, 0, st>>>(y16, y16_scale, pair_pos, w, k, H,
                                                        n_chunks, items, out, out_f32);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* y_sorted, const int32_t* pair_pos, const float* w, int T,
                           int k, int H, bool out_bf16, void* out, float* out_f32,
                           hipStream_t st) {
  const int n_chunks = (H + FCOLS - 1) / FCOLS;
  const long long items = (long long)T * n_chunks;
  const unsigned grid = (unsigned)(items < (1 << 20) ? items : (1 << 20));
  if (out_bf16)
    finalize_kernel<true><<<grid, 256, 0, st>>>(y_sorted, pair_pos, w, k, H, n_chunks, items, out,
                                                out_f32);
  else
    finalize_kernel<false><<<grid, 256, 0, st>>>(y_sorted, pair_pos, w, k, H, n_chunks, items, out,
                                                 out_f32);
  return hipGetLastError();
}

}  // namespace moe
