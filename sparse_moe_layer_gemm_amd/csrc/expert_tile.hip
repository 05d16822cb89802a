// Grouped SwiGLU expert GEMMs of Beam's routed MoE layer for many rows per
// expert (prefill-sized batches), on gfx950 MFMA.
//
// Same operation as the streaming kernel (per-expert GEMMs with gate and up
// merged, "merged projections", UpstreamBeat "vLLM adds day-zero Reflection
// Beam serving...", section "Agents worked on the serving path"), scheduled
// for the dense-contraction regime:
//  - one workgroup (4 wavefronts) computes a 128-row x 256-column output tile
//    of one expert; each wavefront owns 64 x 128 (4 x 8 MFMA 16x16x32 tiles);
//  - K advances 64 at a time through double-buffered LDS (96 KB): the next
//    K step's global loads are issued before the current step's MFMAs and
//    written to the other buffer afterwards, one barrier per step;
//  - A rows are gathered (token rows of x for gate/up, rows of h for down);
//    B is stored [K, N] (N contiguous), so each thread loads an 8 x 8 block
//    and transposes it in registers into K-contiguous 16-byte granules;
//  - LDS rows are 128 bytes with the 16-byte granule index XOR-swizzled by
//    the row, so the fragment reads of 16 consecutive rows are conflict-free;
//  - for gate/up the tile holds 128 gate columns and the matching 128 up
//    columns, so each lane forms silu(gate) * up from two of its own
//    accumulators;
//  - workgroups map onto (M tile, N tile) so that consecutive work items,
//    which share A rows and B panels, land on the same XCD (and its L2).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TBM = 128, TBN = 256, TBK = 64;
constexpr int TSTAGE_A = TBM * TBK * 2;  // bytes per A stage
constexpr int TSTAGE_B = TBN * TBK * 2;  // bytes per B stage

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Byte offset of 16-byte granule kb (8 K values) of LDS row `row` (128 B rows).
__device__ __forceinline__ int lds_off(int row, int kb) {
  const int g = ((row >> 1) ^ (row >> 3)) & 7;
  return row * 128 + ((kb ^ g) << 4);
}

// M-tile table: tiles of TBM rows per expert, in expert order.
__global__ __launch_bounds__(256) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                         int E, int bm,
                                                         int32_t* __restrict__ tile_e,
                                                         int32_t* __restrict__ tile_m0,
                                                         int32_t* __restrict__ n_tiles) {
  __shared__ int cnt[256];
  const int e = threadIdx.x;
  const int c = (e < E) ? (offsets[e + 1] - offsets[e] + bm - 1) / bm : 0;
  cnt[e] = c;
  __syncthreads();
  // inclusive scan (Hillis-Steele over 256 entries)
  for (int d = 1; d < 256; d <<= 1) {
    const int v = (e >= d) ? cnt[e - d] : 0;
    __syncthreads();
    cnt[e] += v;
    __syncthreads();
  }
  const int base = cnt[e] - c;
  for (int j = 0; j < c; ++j) {
    tile_e[base + j] = e;
    tile_m0[base + j] = j * bm;
  }
  if (e == 255) *n_tiles = cnt[255];
}

template <bool GATE_UP>
__global__ __launch_bounds__(256, 1) void tile_bf16_kernel(StreamGemmArgs a,
                                                           const int32_t* __restrict__ tile_e,
                                                           const int32_t* __restrict__ tile_m0,
                                                           const int32_t* __restrict__ n_tiles_p,
                                                           int NT) {
  __shared__ __align__(16) uint8_t smem[2 * (TSTAGE_A + TSTAGE_B)];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- work item (XCD-aware: consecutive items on the same XCD)
  const int total = *n_tiles_p * NT;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = (total + 7) >> 3;
  if (slot >= per) return;
  const int w = xcd * per + slot;
  if (w >= total) return;
  const int mt = w / NT, nt = w - mt * NT;
  const int e = tile_e[mt];
  const int m0 = tile_m0[mt];
  const int r0 = a.offsets[e];
  const int cnt = a.offsets[e + 1] - r0;
  const int K = a.K, N = a.N;

  // ---- global load assignments
  // A: thread owns half a row (4 granules) of the 128-row tile
  const int arow = tid >> 1, ahalf = tid & 1;
  const bool a_ok = m0 + arow < cnt;
  const uint16_t* aptr = a.a;
  {
    size_t row = 0;
    if (a_ok) row = GATE_UP ? (size_t)(a.sorted_pair[r0 + m0 + arow] / a.k) : (size_t)(r0 + m0 + arow);
    aptr = a.a + row * K + ahalf * 32;
  }
  // B: thread owns the 8 x 8 block (kb, nb) of the 64 x 256 tile
  const int bkb = tid >> 5, bnb = tid & 31;
  int bcol;  // global column of the block's first column
  if (GATE_UP) {
    const int g0 = nt * (TBN / 2);
    bcol = (bnb < 16) ? g0 + 8 * bnb : a.I + g0 + 8 * (bnb - 16);
  } else {
    bcol = nt * TBN + 8 * bnb;
  }
  const bool b_ok = GATE_UP ? (nt * (TBN / 2) + 8 * (bnb & 15) < a.I) : (bcol < N);
  const uint16_t* bptr = static_cast<const uint16_t*>(a.w) + (size_t)e * K * N + (b_ok ? bcol : 0) +
                         (size_t)(8 * bkb) * N;

  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  u32x4 ra[4], rb[8];
  auto gload = [&](int kt) {
    const int k0 = kt * TBK;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ra[q] = a_ok ? *reinterpret_cast<const u32x4*>(aptr + k0 + 8 * q) : zero;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      rb[r] = b_ok ? *reinterpret_cast<const u32x4*>(bptr + (size_t)(k0 + r) * N) : zero;
  };
  auto lstore = [&](int buf) {
    uint8_t* As = smem + buf * (TSTAGE_A + TSTAGE_B);
    uint8_t* Bs = As + TSTAGE_A;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(As + lds_off(arow, 4 * ahalf + q)) = ra[q];
    // 8 x 8 transpose: column c's 8 K values -> one granule
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u32x4 lo, hi;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t x0 = rb[2 * p][d], x1 = rb[2 * p + 1][d];
        lo[p] = (x0 & 0xFFFFu) | (x1 << 16);
        hi[p] = (x0 >> 16) | (x1 & 0xFFFF0000u);
      }
      *reinterpret_cast<u32x4*>(Bs + lds_off(8 * bnb + 2 * d, bkb)) = lo;
      *reinterpret_cast<u32x4*>(Bs + lds_off(8 * bnb + 2 * d + 1, bkb)) = hi;
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS column of this wave's n-tile j
  auto bcol_lds = [&](int j) -> int {
    if (GATE_UP) return (j < 4) ? 64 * wn + 16 * j : 128 + 64 * wn + 16 * (j - 4);
    return 128 * wn + 16 * j;
  };

  const int nk = K / TBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* As = smem + (kt & 1) * (TSTAGE_A + TSTAGE_B);
    const uint8_t* Bs = As + TSTAGE_A;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kb = 4 * s + (lane >> 4);
      u32x4 fa[4], fb[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(As + lds_off(64 * wm + 16 * i + (lane & 15), kb));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(Bs + lds_off(bcol_lds(j) + (lane & 15), kb));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*(lane>>4)+r of column lane&15 of each 16x16 tile
  const int cl = lane & 15, rq = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 64 * wm + 16 * i + rq + r;
      if (m >= cnt) continue;
      const size_t row = (size_t)(r0 + m);
      if (GATE_UP) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * (TBN / 2) + 64 * wn + 16 * j + cl;
          if (col < a.I)
            a.h_out[row * a.I + col] = (uint16_t)f32_to_bf16_bits(silu(acc[i][j][r]) * acc[i][j + 4][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = nt * TBN + 128 * wn + 16 * j + cl;
          if (col < N) a.y_out[row * N + col] = acc[i][j][r];
        }
      }
    }
  }
}

}  // namespace

size_t expert_tile_ws_bytes(int P, int E) {
  const int max_tiles = (P + TBM - 1) / TBM + E;
  return (size_t)(2 * max_tiles + 64) * sizeof(int32_t);
}

hipError_t launch_expert_tile(int wfmt, const StreamGemmArgs& gu, const StreamGemmArgs& dn, int P,
                              void* ws, hipStream_t st) {
  if (wfmt != W_BF16) return hipErrorInvalidValue;
  const int max_tiles = (P + TBM - 1) / TBM + gu.E;
  int32_t* tile_e = static_cast<int32_t*>(ws);
  int32_t* tile_m0 = tile_e + max_tiles;
  int32_t* n_tiles = tile_m0 + max_tiles;
  tile_table_kernel<<<1, 256, 0, st>>>(gu.offsets, gu.E, TBM, tile_e, tile_m0, n_tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    const int NT = (gu.I + TBN / 2 - 1) / (TBN / 2);
    const long long items = (long long)max_tiles * NT;
    const unsigned grid = (unsigned)(((items + 7) / 8) * 8);
    tile_bf16_kernel<true><<<grid, 256, 0, st>>>(gu, tile_e, tile_m0, n_tiles, NT);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const int NT = (dn.N + TBN - 1) / TBN;
    const long long items = (long long)max_tiles * NT;
    const unsigned grid = (unsigned)(((items + 7) / 8) * 8);
    tile_bf16_kernel<false><<<grid, 256, 0, st>>>(dn, tile_e, tile_m0, n_tiles, NT);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moe
