// Router of Beam's routed MoE layer on gfx950: the FP32 GEMM x[T,H] . W_r[H,E]
// with BF16 logits out (vLLM PR #61978, Status table row #62042; UpstreamBeat,
// "Agents worked on the serving path": a specialized FP32 router kernel),
// followed by softmax, top-k (8 of 256 experts per token, recipe Guide >
// Overview) and renormalisation of the chosen weights.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RBM = 64;   // tokens per workgroup
constexpr int RBK = 32;   // K elements per LDS stage
constexpr int XS_LD = RBM + 16;  // LDS row stride of the transposed x tile (conflict-free reads)

// One workgroup = 4 wavefronts = 64 tokens x 256 expert columns (64 per wave)
// over one K slice. fp32 MFMA 16x16x4: the B fragment is one fp32 per lane,
// so W_r rows are read straight from global memory, 4 consecutive columns per
// lane (one float4); the four columns feed four MFMAs whose output columns
// are strided by 4. x is staged through LDS, transposed to [k][token].
template <bool XBF16>
__global__ __launch_bounds__(256) void router_gemm_kernel(const void* __restrict__ xv, int T,
                                                          int H, const float* __restrict__ wr,
                                                          int E, int split_len,
                                                          float* __restrict__ part) {
  __shared__ float xs[RBK][XS_LD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kl = lane >> 4, jl = lane & 15;
  const int m0 = blockIdx.x * RBM;
  const int s = blockIdx.y;
  const int kbeg = s * split_len;
  const int kend = min(H, kbeg + split_len);
  const int c0 = wave * 64 + 4 * jl;  // this lane's first column
  const bool vec_ok = (E % 4) == 0 && c0 + 3 < E;

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lrow = tid >> 2, lk = (tid & 3) * 8;
  const int lt = m0 + lrow;
  for (int k0 = kbeg; k0 < kend; k0 += RBK) {
    float v[8];
    if (lt < T) {
      if constexpr (XBF16) {
        const uint4 q = *reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(xv) + (size_t)lt * H + k0 + lk);
        const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(d[i] << 16);
          v[2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(xv) +
                                                          (size_t)lt * H + k0 + lk);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    __syncthreads();  // previous stage's readers are done
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[lk + i][lrow] = v[i];
    __syncthreads();

    if (wave * 64 < E) {
#pragma unroll 2
      for (int st = 0; st < RBK / 4; ++st) {
        const int kk = k0 + st * 4 + kl;
        const float* wrow = wr + (size_t)kk * E;
        float b[4];
        if (vec_ok) {
          const float4 q = *reinterpret_cast<const float4*>(wrow + c0);
          b[0] = q.x; b[1] = q.y; b[2] = q.z; b[3] = q.w;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) b[q] = (c0 + q < E) ? wrow[c0 + q] : 0.f;
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const float a = xs[st * 4 + kl][rt * 16 + jl];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[rt][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b[q], acc[rt][q], 0, 0, 0);
        }
      }
    }
  }

  // D layout: lane (kl, jl) holds rows 4*kl + r of column jl of each 16x16 tile;
  // MFMA q's column jl is global column c0 + q.
  if (wave * 64 >= E || c0 >= E) return;
  float* dst = part + (size_t)s * T * E;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = m0 + rt * 16 + 4 * kl + r;
      if (t >= T) continue;
      float* o = dst + (size_t)t * E + c0;
      if (vec_ok) {
        *reinterpret_cast<float4*>(o) =
            make_float4(acc[rt][0][r], acc[rt][1][r], acc[rt][2][r], acc[rt][3][r]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c0 + q < E) o[q] = acc[rt][q][r];
      }
    }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// One wavefront per token; lane l holds experts l, l+64, l+128, l+192.
// The selection key packs (order-preserving logit, 0xFFFF - id) so that a
// wave-wide max picks the largest logit and, on equal logits, the lowest id.
template <bool BF16_LOGITS>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ part, int n_split, int ldp, int T, int E, int k,
    const float* __restrict__ bias, void* __restrict__ logits, float* __restrict__ logits_f32,
    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  uint64_t key[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    key[q] = 0;
    if (e < E) {
      float v = 0.f;
      for (int s = 0; s < n_split; ++s) v += part[((size_t)s * T + t) * ldp + e];
      if (bias) v += bias[e];
      if (logits_f32) logits_f32[(size_t)t * E + e] = v;
      float sv = v;
      if constexpr (BF16_LOGITS) {
        const uint32_t b = f32_to_bf16_bits(v);
        static_cast<uint16_t*>(logits)[(size_t)t * E + e] = (uint16_t)b;
        sv = bf16_bits_to_f32(b);
      } else {
        static_cast<float*>(logits)[(size_t)t * E + e] = v;
      }
      key[q] = ((uint64_t)float_order_key(sv) << 32) | (uint32_t)(0xFFFF - e);
    }
  }
  float topv[8];
  int topi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    topv[j] = 0.f;
    topi[j] = 0;
    if (j < k) {
      uint64_t best = key[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) best = key[q] > best ? key[q] : best;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = shfl_xor_u64(best, m);
        best = o > best ? o : best;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (key[q] == best) key[q] = 0;
      topi[j] = 0xFFFF - (int)(best & 0xFFFFu);
      topv[j] = float_from_order_key((uint32_t)(best >> 32));
    }
  }
  if (lane == 0) {
    // softmax over all E, restricted to the chosen set: the normaliser cancels
    float p[8], z = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = (j < k) ? expf(topv[j] - topv[0]) : 0.f;
      z += p[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) {
        ids[(size_t)t * k + j] = topi[j];
        w[(size_t)t * k + j] = p[j] / z;
      }
  }
}

}  // namespace

hipError_t launch_router_gemm(const void* x, bool x_bf16, int T, int H, const float* w_router,
                              int E, int n_split, int split_len, float* part, hipStream_t st) {
  dim3 grid((T + RBM - 1) / RBM, n_split);
  if (x_bf16)
    router_gemm_kernel<true><<<grid, 256, 0, st>>>(x, T, H, w_router, E, split_len, part);
  else
    router_gemm_kernel<false><<<grid, 256, 0, st>>>(x, T, H, w_router, E, split_len, part);
  return hipGetLastError();
}

hipError_t launch_router_select(const float* part, int n_split, int ldp, int T, int E, int k,
                                const float* bias, bool logits_bf16, void* logits,
                                float* logits_f32, int32_t* ids, float* w, hipStream_t st) {
  dim3 grid((T + 3) / 4);
  if (logits_bf16)
    router_select_kernel<true><<<grid, 256, 0, st>>>(part, n_split, ldp, T, E, k, bias, logits,
                                                     logits_f32, ids, w);
  else
    router_select_kernel<false><<<grid, 256, 0, st>>>(part, n_split, ldp, T, E, k, bias, logits,
                                                      logits_f32, ids, w);
  return hipGetLastError();
}

}  // namespace moe
