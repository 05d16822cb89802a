// MoE finalize on gfx950: the weighted un-permute that closes Beam's routed
// MoE layer (vLLM PR #61978, Status table row #62366 and Remaining work name
// it as its own kernel). out[t] = sum_j w[t, j] * y_sorted[pair_pos[t*k + j]],
// fp32 accumulation in slot order, then round-to-nearest-even to bf16.
//
// Bound by HBM: every fp32 expert row is read once and every output row
// written once. One workgroup per token; the k row positions and weights are
// wave-uniform (scalar loads), and each lane streams float4 columns.
#include "moe_internal.h"

namespace moe {
namespace {

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ y,
                                                       const int32_t* __restrict__ pair_pos,
                                                       const float* __restrict__ w, int k, int H,
                                                       void* __restrict__ out,
                                                       float* __restrict__ out_f32) {
  const int t = blockIdx.x;
  int pos[8];
  float wt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pos[j] = (j < k) ? pair_pos[(size_t)t * k + j] : 0;
    wt[j] = (j < k) ? w[(size_t)t * k + j] : 0.f;
  }
  for (int c = threadIdx.x * 4; c < H; c += 256 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      const float4 v = *reinterpret_cast<const float4*>(y + (size_t)pos[j] * H + c);
      acc.x = fmaf(wt[j], v.x, acc.x);
      acc.y = fmaf(wt[j], v.y, acc.y);
      acc.z = fmaf(wt[j], v.z, acc.z);
      acc.w = fmaf(wt[j], v.w, acc.w);
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

}  // namespace

hipError_t launch_finalize(const float* y_sorted, const int32_t* pair_pos, const float* w, int T,
                           int k, int H, bool out_bf16, void* out, float* out_f32,
                           hipStream_t st) {
  if (out_bf16)
    finalize_kernel<true><<<T, 256, 0, st>>>(y_sorted, pair_pos, w, k, H, out, out_f32);
  else
    finalize_kernel<false><<<T, 256, 0, st>>>(y_sorted, pair_pos, w, k, H, out, out_f32);
  return hipGetLastError();
}

}  // namespace moe
