// Token permute by expert on gfx950: histogram, exclusive scan and stable
// scatter of the (token, slot) pairs, so that each expert's rows are
// contiguous for the grouped expert GEMMs and the finalize step can find
// every pair again (vLLM PR #61978: "MoE finalize" is the weighted
// un-permute of these rows, Status table row #62366).
//
// Each wavefront owns a contiguous segment of pairs and keeps its own 256-bin
// histogram in LDS, so no atomics are needed and the result is deterministic:
// ranks within a 64-pair chunk come from a ballot-based match of equal expert
// ids, chunks are walked in order, and segments are ordered by index. Up to
// 16384 pairs one workgroup of 16 wavefronts does it all; above, segments of
// >= 512 pairs spread over many workgroups with a scan kernel between the
// histogram and scatter passes.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int PW = 16;  // wavefronts per workgroup
constexpr int kScanBatch = 16;  // segment counts the scan loads per batch

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
  // ids outside [0, E) have no sorted row: the rows past the last expert's
  // end read -1, and so do those pairs' positions (set in pass 3)
  for (int r = total + tid; r < P; r += 1024) sorted_pair[r] = -1;

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
    } else if (p < s1) {
      pair_pos[p] = -1;
    }
    if (valid && lane == 63 - __builtin_clzll(peers)) hist[wave][id] += __popcll(peers);
  }
}

// Ids of kChunkBatch consecutive 64-pair chunks from c0 on, loaded together
// (one memory latency per batch); pairs at or past s1 read as -1 (invalid).
constexpr int kChunkBatch = 8;
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ ids, int c0, int s1, int lane,
                                         int (&idb)[kChunkBatch]) {
  int raw[kChunkBatch];
#pragma unroll
  for (int b = 0; b < kChunkBatch; ++b) {
    const int p = c0 + 64 * b + lane;
    raw[b] = ids[p < s1 ? p : s1 - 1];  // clamped: every load is in bounds
  }
#pragma unroll
  for (int b = 0; b < kChunkBatch; ++b) idb[b] = (c0 + 64 * b + lane < s1) ? raw[b] : -1;
}

// ---- many pairs: the same per-wavefront algorithm over NV segments spread
// across workgroups. Segment v (wavefront v % 16 of workgroup v / 16) holds
// pairs [v * seg, (v + 1) * seg); its histogram goes to hist_g[v * E + e]
// (segment-major, so every access to hist_g is coalesced across experts), one
// workgroup turns those into scatter starts, and the scatter pass replays the
// same stable ranks.
__global__ __launch_bounds__(1024) void permute_hist_kernel(const int32_t* __restrict__ ids, int P,
                                                            int E, int seg, int NV,
                                                            int32_t* __restrict__ hist_g) {
  __shared__ int hist[PW][256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < PW * 256; i += 1024) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int v = blockIdx.x * PW + wave;
  const long long s0l = (long long)v * seg;
  const int s0 = (int)(s0l < P ? s0l : P), s1 = (int)(s0l + seg < P ? s0l + seg : P);
  for (int c0 = s0; c0 < s1; c0 += 64 * kChunkBatch) {
    int idb[kChunkBatch];
    load_ids(ids, c0, s1, lane, idb);
#pragma unroll
    for (int b = 0; b < kChunkBatch; ++b) {
      int id = idb[b];
      const bool valid = id >= 0 && id < E;
      if (!valid) id = 0;
      const uint64_t peers = match_peers(id, valid);
      if (valid && lane == 63 - __builtin_clzll(peers)) hist[wave][id] += __popcll(peers);
    }
  }
  __syncthreads();
  if (v < NV)
    for (int e = lane; e < E; e += 64) hist_g[(size_t)v * E + e] = hist[wave][e];
}

// One workgroup: for every expert, exclusive prefix of its segment counts in
// segment order, then the scan over experts; hist_g becomes each segment's
// first position. Thread (q, e) takes expert e over the q-th quarter of the
// segments, so a wavefront's loads read 64 adjacent experts of one segment;
// the loads of kScanBatch segments are issued together.
__global__ __launch_bounds__(1024) void permute_scan_kernel(int E, int NV, int32_t* __restrict__ hist_g,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int part[4][256];
  __shared__ int base[256];
  __shared__ int total;
  const int tid = threadIdx.x, q = tid >> 8, e = tid & 255, lane = tid & 63;
  const int per = (NV + 3) / 4;
  const int v0 = min(NV, q * per), v1 = min(NV, v0 + per);
  const bool live = e < E;
  const int ec = live ? e : 0;  // clamped column: every load is in bounds
  int sum = 0;
  for (int vb = v0; vb < v1; vb += kScanBatch) {
    int c[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) c[i] = hist_g[(size_t)(vb + i < v1 ? vb + i : v1 - 1) * E + ec];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (vb + i < v1) sum += c[i];
  }
  part[q][e] = live ? sum : 0;
  __syncthreads();
  if (tid < 256) {
    const int t = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
    base[tid] = t;
    if (tid < E) counts[tid] = t;
  }
  __syncthreads();
  if (tid < 64) {
    // exclusive scan of base[0..256): lane owns 4 consecutive experts
    const int w0 = base[4 * lane], w1 = base[4 * lane + 1], w2 = base[4 * lane + 2],
              w3 = base[4 * lane + 3];
    const int s4 = w0 + w1 + w2 + w3;
    int incl = s4;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int ex = incl - s4;
    if (lane == 63) total = incl;
    base[4 * lane] = ex;
    base[4 * lane + 1] = ex + w0;
    base[4 * lane + 2] = ex + w0 + w1;
    base[4 * lane + 3] = ex + w0 + w1 + w2;
  }
  __syncthreads();
  if (tid < E) offsets[tid] = base[tid];
  if (tid == 0) offsets[E] = total;
  if (!live) return;
  int run = base[e];
  for (int qq = 0; qq < q; ++qq) run += part[qq][e];
  for (int vb = v0; vb < v1; vb += kScanBatch) {
    int c[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) c[i] = hist_g[(size_t)(vb + i < v1 ? vb + i : v1 - 1) * E + e];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (vb + i < v1) {
        hist_g[(size_t)(vb + i) * E + e] = run;
        run += c[i];
      }
  }
}

__global__ __launch_bounds__(1024) void permute_scatter_kernel(const int32_t* __restrict__ ids,
                                                               int P, int E, int seg, int NV,
                                                               const int32_t* __restrict__ hist_g,
                                                               const int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pair,
                                                               int32_t* __restrict__ pair_pos) {
  __shared__ int hist[PW][256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // rows past the last expert's end (pairs with ids outside [0, E)) read -1
  for (long long r = (long long)offsets[E] + (long long)blockIdx.x * 1024 + tid; r < P;
       r += (long long)gridDim.x * 1024)
    sorted_pair[r] = -1;
  const int v = blockIdx.x * PW + wave;
  if (v < NV)
    for (int e = lane; e < E; e += 64) hist[wave][e] = hist_g[(size_t)v * E + e];
  __syncthreads();
  const long long s0l = (long long)v * seg;
  const int s0 = (int)(s0l < P ? s0l : P), s1 = (int)(s0l + seg < P ? s0l + seg : P);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = s0; c0 < s1; c0 += 64 * kChunkBatch) {
    int idb[kChunkBatch];
    load_ids(ids, c0, s1, lane, idb);
#pragma unroll
    for (int b = 0; b < kChunkBatch; ++b) {
      const int p = c0 + 64 * b + lane;
      int id = idb[b];
      const bool valid = id >= 0 && id < E;
      if (!valid) id = 0;
      const uint64_t peers = match_peers(id, valid);
      if (valid) {
        const int pos = hist[wave][id] + __popcll(peers & below);
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
      } else if (p < s1) {
        pair_pos[p] = -1;
      }
      if (valid && lane == 63 - __builtin_clzll(peers)) hist[wave][id] += __popcll(peers);
    }
  }
}

}  // namespace

void permute_plan(long long P, int* seg, int* nv) {
  // segments of at least 512 pairs (8 chunks per wavefront), at most 32768 of them
  long long n = (P + 511) / 512;
  if (n > 32768) n = 32768;
  if (n < 1) n = 1;
  long long s = (P + n - 1) / n;
  s = (s + 63) / 64 * 64;
  *seg = (int)s;
  *nv = (int)((P + s - 1) / s);
}

size_t permute_ws_bytes(long long P, int E) {
  if (P <= kPermuteOneBlockMax) return 0;
  int seg, nv;
  permute_plan(P, &seg, &nv);
  return (size_t)E * nv * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, void* ws, hipStream_t st) {
  if (P <= kPermuteOneBlockMax) {
    permute_kernel<<<1, 1024, 0, st>>>(ids, P, E, counts, offsets, sorted_pair, pair_pos);
    return hipGetLastError();
  }
  int seg, nv;
  permute_plan(P, &seg, &nv);
  int32_t* hist_g = static_cast<int32_t*>(ws);
  const unsigned blocks = (unsigned)((nv + PW - 1) / PW);
  permute_hist_kernel<<<blocks, 1024, 0, st>>>(ids, P, E, seg, nv, hist_g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scan_kernel<<<1, 1024, 0, st>>>(E, nv, hist_g, counts, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scatter_kernel<<<blocks, 1024, 0, st>>>(ids, P, E, seg, nv, hist_g, offsets, sorted_pair,
                                                  pair_pos);
  return hipGetLastError();
}

}  // namespace moe
