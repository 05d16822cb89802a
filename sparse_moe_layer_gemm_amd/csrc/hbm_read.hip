// Measured HBM read ceiling on gfx950: a plain streaming read of a device
// buffer, in the access pattern the decode expert kernels use for weights
// (16-byte nontemporal loads, several in flight per lane, every byte read
// once). The layer's HBM-bound kernels are quoted against its rate as well as
// against the published 8 TB/s.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int HR_THREADS = 256;
constexpr int HR_UNROLL = 8;  // loads in flight per lane

// Workgroup b streams its own contiguous range of the buffer; per iteration
// lane t of the workgroup loads elements base + u * 256 + t for u < 8, so each
// wavefront's load covers 1 KB contiguous and a workgroup's eight cover 32 KB.
__global__ __launch_bounds__(HR_THREADS) void hbm_read_kernel(const u32x4* __restrict__ src,
                                                              long long n, long long per,
                                                              uint32_t* __restrict__ sink) {
  const long long beg = (long long)blockIdx.x * per;
  const long long end = beg + per < n ? beg + per : n;
  long long i = beg + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (HR_UNROLL - 1) * HR_THREADS < end; i += HR_UNROLL * HR_THREADS) {
    u32x4 v[HR_UNROLL];
#pragma unroll
    for (int u = 0; u < HR_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * HR_THREADS);
#pragma unroll
    for (int u = 0; u < HR_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += HR_THREADS) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // keeps the loads live; the store happens only for one XOR value
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  const long long n = (long long)(bytes / 16);
  if (n <= 0) return hipSuccess;
  // 8 workgroups per CU of the 256, each over a contiguous range
  const long long blocks = std::min<long long>(2048, (n + HR_THREADS - 1) / HR_THREADS);
  const long long per = (n + blocks - 1) / blocks;
  hbm_read_kernel<<<(unsigned)blocks, HR_THREADS, 0, st>>>(static_cast<const u32x4*>(buf), n, per,
                                                           sink);
  return hipGetLastError();
}

}  // namespace moe
