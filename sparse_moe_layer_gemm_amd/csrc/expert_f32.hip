// fp32 grouped SwiGLU expert GEMMs: the all-fp32 form of the layer's experts
// (gate = columns [0, I), up = columns [I, 2I) of the merged gate/up matrix,
// h = silu(gate) * up, y = h . W_down). One thread per output element with an
// fp32 dot product over K; used for small all-fp32 layers where exact fp32
// products matter more than throughput.
#include "moe_internal.h"

namespace moe {
namespace {

// Expert owning sorted row r: the e with offsets[e] <= r < offsets[e + 1].
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // invariant: offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void f32_gate_up_kernel(const float* __restrict__ x, int H, int I,
                                                          int E, int k,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_pair,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ h) {
  const int r = blockIdx.x;
  const int i = blockIdx.y * 256 + threadIdx.x;
  if (i >= I || r >= offsets[E]) return;  // rows past the last expert's end have no pair
  const int e = expert_of_row(offsets, E, r);
  const float* xr = x + (size_t)(sorted_pair[r] / k) * H;
  const float* wg = w + (size_t)e * H * 2 * I + i;
  float gv = 0.f, uv = 0.f;
  for (int hh = 0; hh < H; ++hh) {
    const float xv = xr[hh];
    gv = fmaf(xv, wg[(size_t)hh * 2 * I], gv);
    uv = fmaf(xv, wg[(size_t)hh * 2 * I + I], uv);
  }
  h[(size_t)r * I + i] = silu(gv) * uv;
}

__global__ __launch_bounds__(256) void f32_down_kernel(const float* __restrict__ h, int H, int I,
                                                       int E, const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ w,
                                                       float* __restrict__ y) {
  const int r = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (n >= H || r >= offsets[E]) return;
  const int e = expert_of_row(offsets, E, r);
  const float* hr = h + (size_t)r * I;
  const float* wd = w + (size_t)e * I * H + n;
  float acc = 0.f;
  for (int i = 0; i < I; ++i) acc = fmaf(hr[i], wd[(size_t)i * H], acc);
  y[(size_t)r * H + n] = acc;
}

}  // namespace

hipError_t launch_expert_f32(const float* x, int T, int H, int I, int E, int k, int P,
                             const int32_t* offsets, const int32_t* sorted_pair,
                             const float* gate_up, const float* down, float* h, float* y,
                             hipStream_t st) {
  (void)T;
  if (P == 0) return hipSuccess;
  f32_gate_up_kernel<<<dim3(P, (I + 255) / 256), 256, 0, st>>>(x, H, I, E, k, offsets, sorted_pair,
                                                                gate_up, h);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  f32_down_kernel<<<dim3(P, (H + 255) / 256), 256, 0, st>>>(h, H, I, E, offsets, down, y);
  return hipGetLastError();
}

}  // namespace moe
