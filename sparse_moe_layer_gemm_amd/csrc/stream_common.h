// Device helpers shared by the streaming expert kernels (few rows per
// expert): the bf16 16x16x32 MFMA and the expert of a grid row.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The expert of grid row `slot`. With one row per expert (gridDim.y == E) it
// is the row itself; with fewer rows (min(E, P) < E: few pairs, so most
// experts are empty) it is the slot-th expert that has rows, found from the
// offsets by ballots (every lane of the wavefront gets the same answer), or
// -1 when fewer experts have rows.
__device__ __forceinline__ int slot_expert(const int32_t* __restrict__ offsets, int E, int slot,
                                           int lane) {
  if ((int)gridDim.y == E) return slot;
  int o0[4], o1[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {  // E <= 256: lane l looks at experts l, l+64, l+128, l+192
    const int e = 64 * c + lane;
    o0[c] = offsets[e < E ? e : 0];
    o1[c] = offsets[e < E ? e + 1 : 0];
  }
  const uint64_t below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bool nz = 64 * c + lane < E && o1[c] > o0[c];
    const uint64_t m = __ballot(nz);
    const int want = slot - base;
    if (want < __popcll(m)) {
      const uint64_t hit = __ballot(nz && __popcll(m & below) == want);
      return 64 * c + __builtin_ctzll(hit);
    }
    base += __popcll(m);
  }
  return -1;
}

}  // namespace
}  // namespace moe
