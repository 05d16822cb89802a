// Token permute by expert on gfx950: histogram, exclusive scan and stable
// scatter of the (token, slot) pairs, so that each expert's rows are
// contiguous for the grouped expert GEMMs and the finalize step can find
// every pair again (vLLM PR #61978: "MoE finalize" is the weighted
// un-permute of these rows, Status table row #62366).
//
// One workgroup of 16 wavefronts. Each wavefront owns a contiguous segment of
// pairs and keeps its own 256-bin histogram in LDS, so no atomics are needed
// and the result is deterministic: ranks within a 64-pair chunk come from a
// ballot-based match of equal expert ids, chunks are walked in order, and
// segments are ordered by wavefront index.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int PW = 16;  // wavefronts per workgroup

// Lanes of this wavefront whose id equals mine (8-bit ids, invalid lanes excluded).
__device__ __forceinline__ uint64_t match_peers(int id, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (id >> b) & 1;
    const uint64_t set = __ballot(bit);
    peers &= bit ? set : ~set;
  }
  return peers;
}

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ ids, int P,
                                                       int E, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted_pair,
                                                       int32_t* __restrict__ pair_pos) {
  __shared__ int hist[PW][256];
  __shared__ int base[256];
  __shared__ int total;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < PW * 256; i += 1024) (&hist[0][0])[i] = 0;
  __syncthreads();

  const int seg = (P + PW - 1) / PW;
  const int s0 = min(P, wave * seg), s1 = min(P, s0 + seg);
  const uint64_t below = (1ull << lane) - 1ull;

  // pass 1: per-wavefront histogram
  for (int c = s0; c < s1; c += 64) {
    const int p = c + lane;
    int id = (p < s1) ? ids[p] : -1;
    const bool valid = id >= 0 && id < E;
    if (!valid) id = 0;
    const uint64_t peers = match_peers(id, valid);
    if (valid && lane == 63 - __builtin_clzll(peers)) hist[wave][id] += __popcll(peers);
  }
  __syncthreads();

  // pass 2: per expert, exclusive prefix over wavefronts; then scan over experts
  if (tid < 256) {
    int run = 0;
    if (tid < E)
      for (int w = 0; w < PW; ++w) {
        const int c = hist[w][tid];
        hist[w][tid] = run;
        run += c;
      }
    base[tid] = run;
    if (tid < E) counts[tid] = run;
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of base[0..256): lane owns 4 consecutive experts
    const int v0 = base[4 * lane], v1 = base[4 * lane + 1], v2 = base[4 * lane + 2],
              v3 = base[4 * lane + 3];
    const int sum = v0 + v1 + v2 + v3;
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int ex = incl - sum;
    if (lane == 63) total = incl;
    base[4 * lane] = ex;
    base[4 * lane + 1] = ex + v0;
    base[4 * lane + 2] = ex + v0 + v1;
    base[4 * lane + 3] = ex + v0 + v1 + v2;
  }
  __syncthreads();
  if (tid < E) {
    offsets[tid] = base[tid];
    for (int w = 0; w < PW; ++w) hist[w][tid] += base[tid];
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();

  // pass 3: stable scatter
  for (int c = s0; c < s1; c += 64) {
    const int p = c + lane;
    int id = (p < s1) ? ids[p] : -1;
    const bool valid = id >= 0 && id < E;
    if (!valid) id = 0;
    const uint64_t peers = match_peers(id, valid);
    if (valid) {
      const int pos = hist[wave][id] + __popcll(peers & below);
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    }
    if (valid && lane == 63 - __builtin_clzll(peers)) hist[wave][id] += __popcll(peers);
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, hipStream_t st) {
  permute_kernel<<<1, 1024, 0, st>>>(ids, P, E, counts, offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
