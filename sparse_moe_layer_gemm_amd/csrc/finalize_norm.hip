// MoE finalize fused with the sandwich norms around Beam's routed MoE block
// (vLLM PR #61978, Status table row #62366 fuses the all-reduce with Beam's
// sandwich norms and MoE finalize; on one GPU there is no all-reduce). The
// pages do not define the norm: RMSNorm with a bf16 weight vector, a bf16
// residual stream and a caller-given epsilon are this library's conventions.
// Per token row t:
//   m      = sum_j w[t, j] * y_sorted[pair_pos[t*k + j]]    fp32, slot order
//   post   = m * (1 / sqrt(mean(m^2) + eps)) * gamma_post
//   r      = RNE_bf16(residual + post)                       the new residual
//   normed = RNE_bf16(r * (1 / sqrt(mean(r^2) + eps)) * gamma_next)
//
// Bound by HBM like the plain finalize (each expert row is read once, as fp32
// rows or as compact rows: fp16 with a power-of-two scale per 64 columns).
// Both mean squares need the whole row, so one workgroup owns a token: lane l
// keeps float4 column chunks l, l + NT, ... of m (and then of r) in
// registers, the row sums go through a fixed butterfly in each wavefront and a
// fixed-order add of the wavefront sums, so results are deterministic. Small
// batches use 1024 lanes per token (16 wavefronts: enough loads in flight per
// token); from 1024 tokens on, 256 lanes per token, so that a CU holds four
// times as many tokens and keeps loading while some of them reduce.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kLargeBatch = 1024;  // tokens from which 256 lanes serve a token

// sum over the workgroup of NT lanes, identical in every lane
template <int NT>
__device__ __forceinline__ float row_sum(float v, float* red) {
  constexpr int NWV = NT / 64;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);  // a + b == b + a: lanes agree
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s[NWV];
#pragma unroll
  for (int w = 0; w < NWV; ++w) s[w] = red[w];
#pragma unroll
  for (int d = 1; d < NWV; d <<= 1)  // fixed pairwise order
#pragma unroll
    for (int w = 0; w < NWV; w += 2 * d) s[w] += s[w + d];
  __syncthreads();  // red is reused by the next sum
  return s[0];
}

__device__ __forceinline__ float4 bf16x4_to_f32(uint2 b) {
  return make_float4(bf16_bits_to_f32(b.x & 0xffffu), bf16_bits_to_f32(b.x >> 16),
                     bf16_bits_to_f32(b.y & 0xffffu), bf16_bits_to_f32(b.y >> 16));
}
__device__ __forceinline__ uint2 f32x4_to_bf16(float a, float b, float c, float d) {
  uint2 r;
  r.x = f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
  r.y = f32_to_bf16_bits(c) | (f32_to_bf16_bits(d) << 16);
  return r;
}

// Expert rows the kernel reads: fp32 rows, or compact rows (fp16 values with
// one power-of-two scale byte per row and 64-column block, decoded exactly).
struct NormRows {
  const float* y = nullptr;       // [P, H] fp32
  const uint16_t* y16 = nullptr;  // [P, H] fp16 bits
  const uint8_t* ysc = nullptr;   // [P, H / 64] scale bytes (2^(b - 127))
};

// Float4 chunk q (columns 4q .. 4q + 3) of expert row `pos`.
template <bool R16>
__device__ __forceinline__ f32x4 load_row4(const NormRows& rows, int pos, int H, int q) {
  if constexpr (R16) {
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    const u32x2v v = __builtin_nontemporal_load(
        reinterpret_cast<const u32x2v*>(rows.y16 + (size_t)pos * H) + q);
    const int e = (int)rows.ysc[(size_t)pos * (H >> 6) + (q >> 4)] - 127;
    return f32x4{__builtin_ldexpf(f16_bits_to_f32(v.x & 0xffffu), e),
                 __builtin_ldexpf(f16_bits_to_f32(v.x >> 16), e),
                 __builtin_ldexpf(f16_bits_to_f32(v.y & 0xffffu), e),
                 __builtin_ldexpf(f16_bits_to_f32(v.y >> 16), e)};
  } else {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(rows.y + (size_t)pos * H) + q);
  }
}

// NT lanes per token, CH float4 chunks per lane: H <= 4 * NT * CH. residual and
// residual_out may alias (a lane reads each of its residual chunks before
// writing the same chunk).
template <int NT, int CH, bool R16>
__global__ __launch_bounds__(NT) void finalize_norm_kernel(
    NormRows rows, const int32_t* __restrict__ pair_pos, const float* __restrict__ w,
    int k, int H, const uint16_t* residual, const uint16_t* __restrict__ gamma_post,
    const uint16_t* __restrict__ gamma_next, float eps, uint16_t* residual_out,
    uint16_t* __restrict__ normed) {
  __shared__ float red[NT / 64];
  const long long t = blockIdx.x;
  int pos[8];
  float wt[8];
  bool use[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // wave-uniform; slots past k, and pairs without a row
    const int p = pair_pos[t * k + (j < k ? j : 0)];  // (position -1), read row 0, not added
    use[j] = j < k && p >= 0;
    pos[j] = use[j] ? p : 0;
    wt[j] = use[j] ? w[t * k + j] : 0.f;
  }
  const int n4 = H >> 2;
  float4 m[CH];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int q = threadIdx.x + NT * c;
    m[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (q < n4) {
      f32x4 v[8];  // each expert row is read once: nontemporal
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = load_row4<R16>(rows, pos[j], H, q);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (use[j]) {
          m[c].x = fmaf(wt[j], v[j].x, m[c].x);
          m[c].y = fmaf(wt[j], v[j].y, m[c].y);
          m[c].z = fmaf(wt[j], v[j].z, m[c].z);
          m[c].w = fmaf(wt[j], v[j].w, m[c].w);
        }
      }
      ss += (m[c].x * m[c].x + m[c].y * m[c].y) + (m[c].z * m[c].z + m[c].w * m[c].w);
    }
  }
  const float inv_m = 1.0f / sqrtf(row_sum<NT>(ss, red) / (float)H + eps);
  float ss2 = 0.f;
  const size_t row = (size_t)t * H;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int q = threadIdx.x + NT * c;
    if (q < n4) {
      const float4 res = bf16x4_to_f32(reinterpret_cast<const uint2*>(residual + row)[q]);
      const float4 gp = bf16x4_to_f32(reinterpret_cast<const uint2*>(gamma_post)[q]);
      const uint2 rb = f32x4_to_bf16(res.x + m[c].x * inv_m * gp.x, res.y + m[c].y * inv_m * gp.y,
                                     res.z + m[c].z * inv_m * gp.z, res.w + m[c].w * inv_m * gp.w);
      reinterpret_cast<uint2*>(residual_out + row)[q] = rb;
      m[c] = bf16x4_to_f32(rb);  // from here on m holds r
      ss2 += (m[c].x * m[c].x + m[c].y * m[c].y) + (m[c].z * m[c].z + m[c].w * m[c].w);
    }
  }
  const float inv_r = 1.0f / sqrtf(row_sum<NT>(ss2, red) / (float)H + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int q = threadIdx.x + NT * c;
    if (q < n4) {
      const float4 gn = bf16x4_to_f32(reinterpret_cast<const uint2*>(gamma_next)[q]);
      reinterpret_cast<uint2*>(normed + row)[q] =
          f32x4_to_bf16(m[c].x * inv_r * gn.x, m[c].y * inv_r * gn.y, m[c].z * inv_r * gn.z,
                        m[c].w * inv_r * gn.w);
    }
  }
}

template <int NT, int CH, bool R16>
hipError_t launch_ch(const NormRows& rows, const int32_t* pp, const float* w, int T, int k, int H,
                     const uint16_t* res, const uint16_t* gp, const uint16_t* gn, float eps,
                     uint16_t* res_out, uint16_t* normed, hipStream_t st) {
  finalize_norm_kernel<NT, CH, R16><<<(unsigned)T, NT, 0, st>>>(rows, pp, w, k, H, res, gp, gn,
                                                                eps, res_out, normed);
  return hipGetLastError();
}

template <bool R16>
hipError_t launch_rows(const NormRows& rows, const int32_t* pair_pos, const float* w, int T, int k,
                       int H, const uint16_t* residual, const uint16_t* gamma_post,
                       const uint16_t* gamma_next, float eps, uint16_t* residual_out,
                       uint16_t* normed, hipStream_t st) {
#define MOE_FN_CASE(nt, n)                                                                        \
  case n:                                                                                        \
    return launch_ch<nt, n, R16>(rows, pair_pos, w, T, k, H, residual, gamma_post, gamma_next, eps, \
                                 residual_out, normed, st)
  if (T >= kLargeBatch && H <= 4 * 256 * 6) {
    switch ((H + 4 * 256 - 1) / (4 * 256)) {
      MOE_FN_CASE(256, 1); MOE_FN_CASE(256, 2); MOE_FN_CASE(256, 3); MOE_FN_CASE(256, 4);
      MOE_FN_CASE(256, 5); MOE_FN_CASE(256, 6);
      default:
        return hipErrorInvalidValue;
    }
  }
  switch ((H + 4 * 1024 - 1) / (4 * 1024)) {
    MOE_FN_CASE(1024, 1); MOE_FN_CASE(1024, 2); MOE_FN_CASE(1024, 3); MOE_FN_CASE(1024, 4);
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_FN_CASE
}

}  // namespace

hipError_t launch_finalize_norm(const float* y_sorted, const int32_t* pair_pos, const float* w,
                                int T, int k, int H, const uint16_t* residual,
                                const uint16_t* gamma_post, const uint16_t* gamma_next, float eps,
                                uint16_t* residual_out, uint16_t* normed, hipStream_t st) {
  NormRows rows;
  rows.y = y_sorted;
  return launch_rows<false>(rows, pair_pos, w, T, k, H, residual, gamma_post, gamma_next, eps,
                            residual_out, normed, st);
}

hipError_t launch_finalize_norm_rows16(const uint16_t* y16, const uint8_t* y16_scale,
                                       const int32_t* pair_pos, const float* w, int T, int k,
                                       int H, const uint16_t* residual, const uint16_t* gamma_post,
                                       const uint16_t* gamma_next, float eps,
                                       uint16_t* residual_out, uint16_t* normed, hipStream_t st) {
  NormRows rows;
  rows.y16 = y16;
  rows.ysc = y16_scale;
  return launch_rows<true>(rows, pair_pos, w, T, k, H, residual, gamma_post, gamma_next, eps,
                           residual_out, normed, st);
}

}  // namespace moe
