// Router of Beam's routed MoE layer on gfx950: the FP32 GEMM x[T,H] . W_r[H,E]
// with BF16 logits out (vLLM PR #61978, Status table row #62042; UpstreamBeat,
// "Agents worked on the serving path": a specialized FP32 router kernel),
// followed by softmax, top-k (8 of 256 experts per token, recipe Guide >
// Overview) and renormalisation of the chosen weights.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RBN = 64;  // experts per workgroup
constexpr int RBK = 32;  // K per step

// One workgroup computes a (16 MI)-token x 64-expert block of partial logits
// over one K slice (MI = 1 for batches of at most 16 tokens, whose MFMA work
// would otherwise be padded to 64 rows, else 4); its four wavefronts take the slice's 32-deep steps in turn and
// their sums are added in LDS in wave order. fp32 MFMA 16x16x4 with both
// operands loaded straight into registers, one step ahead: in MFMA s of a step,
// lane group g supplies k = k0 + 8g + s, so a lane's A values for the step are
// 8 consecutive x elements (one 16-byte load for bf16) and its B values are
// rows k0 + 8g + s of W_r at 4 consecutive columns (one float4 each); the four
// columns feed four MFMAs whose output columns are strided by 4.
template <bool XBF16, int MI>
__global__ __launch_bounds__(256) void router_gemm_kernel(const void* __restrict__ xv, int T,
                                                          int H, const float* __restrict__ wr,
                                                          int E, int split_len,
                                                          float* __restrict__ part) {
  __shared__ f32x4 red[4][4 * MI][64];  // per wave: 4 MI accumulator tiles x 64 lanes
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, jl = lane & 15;
  const int m0 = blockIdx.x * 16 * MI, n0 = blockIdx.z * RBN;
  const int s = blockIdx.y;
  const int kbeg = s * split_len;
  const int kend = min(H, kbeg + split_len);
  const int c0 = n0 + 4 * jl;  // this lane's first column
  const bool col_ok = c0 < E;
  const bool vec_ok = (E % 4) == 0 && c0 + 3 < E;

  f32x4 acc[MI][4];
#pragma unroll
  for (int a = 0; a < MI; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A rows of this lane (rows past T read row 0; their results are never stored)
  int arow[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) arow[i] = m0 + 16 * i + jl < T ? m0 + 16 * i + jl : 0;
  float xa[MI][8], xn[MI][8];
  float4 wa[8], wn[8];
  auto load = [&](int k0, float (&xd)[MI][8], float4 (&wd)[8]) {
    const int kk = k0 + 8 * g;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if constexpr (XBF16) {
        const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) +
                                                        (size_t)arow[i] * H + kk);
        const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xd[i][2 * e] = __uint_as_float(d[e] << 16);
          xd[i][2 * e + 1] = __uint_as_float(d[e] & 0xFFFF0000u);
        }
      } else {
        const float4* p =
            reinterpret_cast<const float4*>(static_cast<const float*>(xv) + (size_t)arow[i] * H + kk);
        const float4 u = p[0], v = p[1];
        xd[i][0] = u.x; xd[i][1] = u.y; xd[i][2] = u.z; xd[i][3] = u.w;
        xd[i][4] = v.x; xd[i][5] = v.y; xd[i][6] = v.z; xd[i][7] = v.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float* wrow = wr + (size_t)(kk + e) * E;
      if (vec_ok) {
        wd[e] = *reinterpret_cast<const float4*>(wrow + c0);
      } else {
        wd[e].x = (c0 < E) ? wrow[c0] : 0.f;
        wd[e].y = (c0 + 1 < E) ? wrow[c0 + 1] : 0.f;
        wd[e].z = (c0 + 2 < E) ? wrow[c0 + 2] : 0.f;
        wd[e].w = (c0 + 3 < E) ? wrow[c0 + 3] : 0.f;
      }
    }
  };

  int k0 = kbeg + wave * RBK;
  if (k0 < kend) {
    load(k0, xa, wa);
    for (; k0 < kend; k0 += 4 * RBK) {
      const int kn = (k0 + 4 * RBK < kend) ? k0 + 4 * RBK : k0;  // last step reloads itself
      load(kn, xn, wn);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float b[4] = {wa[e].x, wa[e].y, wa[e].z, wa[e].w};
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[i][e], b[q], acc[i][q], 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        wa[e] = wn[e];
#pragma unroll
        for (int i = 0; i < MI; ++i) xa[i][e] = xn[i][e];
      }
    }
  }

  // add the four wavefronts' sums in wave order
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][4 * i + q][lane] = acc[i][q];
  __syncthreads();
  // thread (wave, lane) finishes tiles 4*wave .. 4*wave+3 of lane `lane`
  // (row group i = wave; waves past the MI row groups have none)
  // D layout: lane (g, jl) holds rows 4g + r of column jl of each 16x16 tile;
  // tile (i, q)'s column jl is global column c0 + q.
  const int i = wave;
  if (i >= MI) return;
  f32x4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = red[0][4 * i + q][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v[q] += red[w][4 * i + q][lane];
  }
  if (!col_ok) return;
  float* dst = part + (size_t)s * T * E;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = m0 + 16 * i + 4 * g + r;
    if (t >= T) continue;
    float* o = dst + (size_t)t * E + c0;
    if (vec_ok) {
      *reinterpret_cast<float4*>(o) = make_float4(v[0][r], v[1][r], v[2][r], v[3][r]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c0 + q < E) o[q] = v[q][r];
    }
  }
}

}  // namespace
}  // namespace moe

// Wavefront-wide maxima of 64- and 32-bit keys (ROCm device library, DPP row
// operations; the result is the same in every lane).
extern "C" __device__ __attribute__((const)) unsigned long long __ockl_wfred_max_u64(
    unsigned long long);
extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_max_u32(unsigned int);

namespace moe {
namespace {

__device__ __forceinline__ uint64_t wave_max(uint64_t v) {
  return (uint64_t)__ockl_wfred_max_u64((unsigned long long)v);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) { return __ockl_wfred_max_u32(v); }

// Selection keys: (order-preserving logit, 0xFFFF - id), so that a maximum is
// the largest logit and, on equal logits, the lowest id. A bf16 logit's order
// key has nothing in its low 16 bits, so with bf16 logits the key is 32 bits
// (the wavefront maxima then compare one register instead of two).
template <bool BF16_LOGITS>
struct SelKey {
  typedef uint64_t type;
  static __device__ __forceinline__ type make(float v, int e) {
    return ((uint64_t)float_order_key(v) << 32) | (uint32_t)(0xFFFF - e);
  }
  static __device__ __forceinline__ float value(type k) { return float_from_order_key((uint32_t)(k >> 32)); }
  static __device__ __forceinline__ int id(type k) { return 0xFFFF - (int)(k & 0xFFFFu); }
};
template <>
struct SelKey<true> {
  typedef uint32_t type;
  static __device__ __forceinline__ type make(float v, int e) {  // v: a bf16 value
    return (float_order_key(v) & 0xFFFF0000u) | (uint32_t)(0xFFFF - e);
  }
  static __device__ __forceinline__ float value(type k) {
    return float_from_order_key((k & 0xFFFF0000u) | ((k & 0x80000000u) ? 0u : 0xFFFFu));
  }
  static __device__ __forceinline__ int id(type k) { return 0xFFFF - (int)(k & 0xFFFFu); }
};

// Small batches (T < 1024, where the router GEMM splits K up to 40 ways):
// one workgroup per token; wavefront w owns experts 64w .. 64w+63, one per
// lane, and adds that expert's split partials (loaded 32 at a time),
// the bias, and rounds to the logits dtype (keys as above). Each wavefront
// finds its own 8 largest
// keys (eight wavefront-wide maxima); wavefront 0 merges the 32 candidates
// into the token's top k.
template <bool BF16_LOGITS>
__global__ __launch_bounds__(256) void router_select_wg_kernel(
    const float* __restrict__ part, int n_split, int ldp, int T, int E, int k,
    const float* __restrict__ bias, void* __restrict__ logits, float* __restrict__ logits_f32,
    int32_t* __restrict__ ids, float* __restrict__ w, PermuteOut perm) {
  using SK = SelKey<BF16_LOGITS>;
  using Key = typename SK::type;
  __shared__ Key cand[4][8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int e = 64 * wave + lane;
  Key key = 0;
  if (e < E) {
    const float* p = part + (size_t)t * ldp + e;
    const size_t sstride = (size_t)T * ldp;
    // the bias goes out with the partials: the same memory latency
    const float be = bias ? bias[e] : 0.f;
    // up to 40 partials (the most the split plan makes) are loaded in one
    // batch (one memory latency), then added in split order
    float v = 0.f;
    for (int sp0 = 0; sp0 < n_split; sp0 += 40) {
      float u[40];
#pragma unroll
      for (int j = 0; j < 40; ++j)
        if (sp0 + j < n_split) u[j] = p[(size_t)(sp0 + j) * sstride];
#pragma unroll
      for (int j = 0; j < 40; ++j)
        if (sp0 + j < n_split) v += u[j];
    }
    if (bias) v += be;
    if (logits_f32) logits_f32[(size_t)t * E + e] = v;
    float sv = v;
    if constexpr (BF16_LOGITS) {
      const uint32_t b = f32_to_bf16_bits(v);
      static_cast<uint16_t*>(logits)[(size_t)t * E + e] = (uint16_t)b;
      sv = bf16_bits_to_f32(b);
    } else {
      static_cast<float*>(logits)[(size_t)t * E + e] = v;
    }
    key = SK::make(sv, e);
  }
  // this wavefront's 8 largest keys, in decreasing order (0 where it has fewer)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const Key best = wave_max(key);
    if (key == best) key = 0;
    if (lane == 0) cand[wave][j] = best;
  }
  __syncthreads();
  if (wave != 0) return;
  Key c = (lane < 32) ? cand[lane >> 3][lane & 7] : (Key)0;
  float topv[8];
  int topi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const Key best = wave_max(c);
    if (c == best) c = 0;
    topi[j] = SK::id(best);
    topv[j] = SK::value(best);
  }
  if (lane == 0) {
    // softmax over all E, restricted to the chosen set: the normaliser cancels
    float pr[8], z = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pr[j] = (j < k) ? expf(topv[j] - topv[0]) : 0.f;
      z += pr[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) {
        ids[(size_t)t * k + j] = topi[j];
        w[(size_t)t * k + j] = pr[j] / z;
      }
  }
  if (perm.counts) {
    // a single token (launched only for T == 1): its k experts are distinct,
    // so the stable sort of its pairs by expert is the rank of each id among
    // the k (topi is the same in every lane of this wavefront)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ex = 64 * c + lane;
      if (ex < E) {
        int below = 0, hit = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < k) {
            below += topi[j] < ex;
            hit |= topi[j] == ex;
          }
        perm.counts[ex] = hit;
        perm.offsets[ex] = below;
      }
    }
    if (lane == 0) perm.offsets[E] = k;
    int mine = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j == lane) mine = topi[j];
    if (lane < k) {
      int pos = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k) pos += topi[j] < mine;
      perm.sorted_pair[pos] = lane;
      perm.pair_pos[lane] = pos;
    }
  }
}

// Large batches: one wavefront per token, four tokens per workgroup. Lane l owns experts
// l, l + 64, l + 128 and l + 192 (coalesced rows), adds each one's split
// partials in split order (loaded SB splits at a time, one memory latency per
// batch; SB covers the split count up to 32), the bias, and rounds to the
// logits dtype. Keys (as above) are distinct. Each of the k
// rounds takes every lane's largest remaining key, their wavefront maximum
// (DPP), and clears it in the lane that holds it: no LDS, no barrier.
template <bool BF16_LOGITS, int SB>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ part, int n_split, int ldp, int T, int E, int k,
    const float* __restrict__ bias, void* __restrict__ logits, float* __restrict__ logits_f32,
    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const float* p = part + (size_t)t * ldp;
  const size_t sstride = (size_t)T * ldp;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp0 = 0; sp0 < n_split; sp0 += SB) {
    float u[4][SB];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if (lane + 64 * q < E && sp0 + j < n_split) u[q][j] = p[(size_t)(sp0 + j) * sstride + lane + 64 * q];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if (lane + 64 * q < E && sp0 + j < n_split) v[q] += u[q][j];
  }
  using SK = SelKey<BF16_LOGITS>;
  using Key = typename SK::type;
  Key key[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    key[q] = 0;
    if (e < E) {
      float x = v[q];
      if (bias) x += bias[e];
      if (logits_f32) logits_f32[(size_t)t * E + e] = x;
      float sv = x;
      if constexpr (BF16_LOGITS) {
        const uint32_t b = f32_to_bf16_bits(x);
        static_cast<uint16_t*>(logits)[(size_t)t * E + e] = (uint16_t)b;
        sv = bf16_bits_to_f32(b);
      } else {
        static_cast<float*>(logits)[(size_t)t * E + e] = x;
      }
      key[q] = SK::make(sv, e);
    }
  }
  float topv[8];
  int topi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    topv[j] = 0.f;
    topi[j] = 0;
    if (j < k) {
      const Key m01 = key[0] > key[1] ? key[0] : key[1];
      const Key m23 = key[2] > key[3] ? key[2] : key[3];
      const Key best = wave_max(m01 > m23 ? m01 : m23);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (key[q] == best) key[q] = 0;
      topi[j] = SK::id(best);
      topv[j] = SK::value(best);
    }
  }
  if (lane == 0) {
    // softmax over all E, restricted to the chosen set: the normaliser cancels
    float pr[8], z = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pr[j] = (j < k) ? expf(topv[j] - topv[0]) : 0.f;
      z += pr[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) {
        ids[(size_t)t * k + j] = topi[j];
        w[(size_t)t * k + j] = pr[j] / z;
      }
  }
}

}  // namespace

int router_gemm_rows(int T) { return T <= 16 ? 16 : 64; }

hipError_t launch_router_gemm(const void* x, bool x_bf16, int T, int H, const float* w_router,
                              int E, int n_split, int split_len, float* part, hipStream_t st) {
  const int rows = router_gemm_rows(T);
  dim3 grid((T + rows - 1) / rows, n_split, (E + RBN - 1) / RBN);
  if (rows == 16) {
    if (x_bf16)
      router_gemm_kernel<true, 1><<<grid, 256, 0, st>>>(x, T, H, w_router, E, split_len, part);
    else
      router_gemm_kernel<false, 1><<<grid, 256, 0, st>>>(x, T, H, w_router, E, split_len, part);
  } else {
    if (x_bf16)
      router_gemm_kernel<true, 4><<<grid, 256, 0, st>>>(x, T, H, w_router, E, split_len, part);
    else
      router_gemm_kernel<false, 4><<<grid, 256, 0, st>>>(x, T, H, w_router, E, split_len, part);
  }
  return hipGetLastError();
}

hipError_t launch_router_select(const float* part, int n_split, int ldp, int T, int E, int k,
                                const float* bias, bool logits_bf16, void* logits,
                                float* logits_f32, int32_t* ids, float* w, hipStream_t st,
                                const PermuteOut* perm) {
  if (perm && T != 1) return hipErrorInvalidValue;
  const PermuteOut po = perm ? *perm : PermuteOut{};
  if (T < 1024) {  // one workgroup per token: 4x the load parallelism per token
    if (logits_bf16)
      router_select_wg_kernel<true><<<T, 256, 0, st>>>(part, n_split, ldp, T, E, k, bias, logits,
                                                       logits_f32, ids, w, po);
    else
      router_select_wg_kernel<false><<<T, 256, 0, st>>>(part, n_split, ldp, T, E, k, bias, logits,
                                                        logits_f32, ids, w, po);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((T + 3) / 4);  // one wavefront per token
#define MOE_SELECT(SB)                                                                         \
  (logits_bf16 ? (router_select_kernel<true, SB><<<grid, 256, 0, st>>>(                         \
                      part, n_split, ldp, T, E, k, bias, logits, logits_f32, ids, w),          \
                  0)                                                                           \
               : (router_select_kernel<false, SB><<<grid, 256, 0, st>>>(                        \
                      part, n_split, ldp, T, E, k, bias, logits, logits_f32, ids, w),          \
                  0))
  if (n_split <= 8)
    MOE_SELECT(8);
  else if (n_split <= 16)
    MOE_SELECT(16);
  else
    MOE_SELECT(32);
#undef MOE_SELECT
  return hipGetLastError();
}

}  // namespace moe
