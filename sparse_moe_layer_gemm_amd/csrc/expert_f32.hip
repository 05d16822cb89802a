// fp32 grouped SwiGLU expert GEMMs: the all-fp32 form of the layer's experts
// (gate = columns [0, I), up = columns [I, 2I) of the merged gate/up matrix,
// h = silu(gate) * up kept in fp32, y = h . W_down), on the fp32 MFMA
// v_mfma_f32_16x16x4_f32: fp32 products, fp32 accumulation.
//
// A workgroup owns one expert and 64 output columns (16 per wavefront) and
// walks the expert's rows 16 at a time; per K step of 4 a lane supplies one A
// value (row l % 16, K index l / 16) and one B value (column l % 16, same K
// index), so the 16 lanes of a K index read 64 contiguous bytes of a weight
// row. Eight K steps of loads are issued before their MFMAs. The result lane l
// holds rows 4 (l / 16) + i of column l % 16.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int F32_UNROLL = 8;  // K steps of 4 whose loads are issued together

// gate/up: every wavefront forms 16 columns of h from its 16 gate and the
// matching 16 up columns (two MFMAs per K step)
__global__ __launch_bounds__(256) void f32_gate_up_kernel(const float* __restrict__ x, int H, int I,
                                                          int k, const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_pair,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ h) {
  const int e = blockIdx.y;
  const int r0 = offsets[e];
  const int cnt = offsets[e + 1] - r0;
  if (cnt <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kg = lane >> 4, cl = lane & 15;
  const int col = blockIdx.x * 64 + 16 * wave + cl;  // < I: I is a multiple of 64
  const float* wg = w + (size_t)e * H * 2 * I + col;
  for (int mc = 0; mc < cnt; mc += 16) {
    // A row of this lane (rows past the expert's end read its first row; their
    // results are never stored)
    const int m = mc + cl;
    const float* xr = x + (size_t)(sorted_pair[r0 + (m < cnt ? m : 0)] / k) * H;
    f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
    for (int k0 = 0; k0 < H; k0 += 4 * F32_UNROLL) {
      float av[F32_UNROLL], gv[F32_UNROLL], uv[F32_UNROLL];
#pragma unroll
      for (int u = 0; u < F32_UNROLL; ++u) {
        const int kk = k0 + 4 * u + kg;
        av[u] = xr[kk];
        gv[u] = wg[(size_t)kk * 2 * I];
        uv[u] = wg[(size_t)kk * 2 * I + I];
      }
#pragma unroll
      for (int u = 0; u < F32_UNROLL; ++u) {
        ag = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], gv[u], ag, 0, 0, 0);
        au = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], uv[u], au, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mc + 4 * kg + i;
      if (row < cnt) h[(size_t)(r0 + row) * I + col] = silu(ag[i]) * au[i];
    }
  }
}

// down: every wavefront forms 16 columns of the expert rows y
__global__ __launch_bounds__(256) void f32_down_kernel(const float* __restrict__ h, int H, int I,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ w,
                                                       float* __restrict__ y) {
  const int e = blockIdx.y;
  const int r0 = offsets[e];
  const int cnt = offsets[e + 1] - r0;
  if (cnt <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kg = lane >> 4, cl = lane & 15;
  const int n = blockIdx.x * 64 + 16 * wave + cl;  // < H: H is a multiple of 64
  const float* wd = w + (size_t)e * I * H + n;
  for (int mc = 0; mc < cnt; mc += 16) {
    const int m = mc + cl;
    const float* hr = h + (size_t)(r0 + (m < cnt ? m : 0)) * I;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < I; k0 += 4 * F32_UNROLL) {
      float av[F32_UNROLL], bv[F32_UNROLL];
#pragma unroll
      for (int u = 0; u < F32_UNROLL; ++u) {
        const int kk = k0 + 4 * u + kg;
        av[u] = hr[kk];
        bv[u] = wd[(size_t)kk * H];
      }
#pragma unroll
      for (int u = 0; u < F32_UNROLL; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], bv[u], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mc + 4 * kg + i;
      if (row < cnt) y[(size_t)(r0 + row) * H + n] = acc[i];
    }
  }
}

}  // namespace

hipError_t launch_expert_f32(const float* x, int T, int H, int I, int E, int k, int P,
                             const int32_t* offsets, const int32_t* sorted_pair,
                             const float* gate_up, const float* down, float* h, float* y,
                             hipStream_t st) {
  (void)T;
  if (P == 0) return hipSuccess;
  // the 64-column workgroups and 32-deep K groups need these multiples (the
  // entry points admit only such shapes)
  if (H % 64 != 0 || I % 64 != 0) return hipErrorInvalidValue;
  f32_gate_up_kernel<<<dim3(I / 64, E), 256, 0, st>>>(x, H, I, k, offsets, sorted_pair, gate_up, h);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  f32_down_kernel<<<dim3(H / 64, E), 256, 0, st>>>(h, H, I, offsets, down, y);
  return hipGetLastError();
}

}  // namespace moe
