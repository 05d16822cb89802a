// Grouped SwiGLU expert GEMMs of Beam's routed MoE layer for many rows per
// expert (prefill-sized batches), on gfx950 MFMA.
//
// Same operation as the streaming kernel (per-expert GEMMs with gate and up
// merged, "merged projections", UpstreamBeat "vLLM adds day-zero Reflection
// Beam serving...", section "Agents worked on the serving path"), scheduled
// for the dense-contraction regime, where the budget that matters is LDS
// bandwidth per MFMA:
//  - one workgroup computes a 256 x 256 output tile of one expert on MFMA
//    32x32x16 (twice the issue rate of 16x16x32 on gfx950). The expert
//    launch runs 8 wavefronts (2 x 4), each owning 128 x 64 (4 x 2 MFMA
//    tiles, 128 fp32 accumulators), two per SIMD; the router's split-bf16
//    GEMM runs 4 wavefronts (2 x 2) of 128 x 128 (256 accumulators, one per
//    SIMD), which halves LDS reads per MFMA. Both measured the same: under
//    sustained MFMA load the chip runs at ~1.55 GHz, and the down GEMM also
//    pays for its fp32 output rows;
//  - an expert's last partial tile of at most 128 rows runs instead as a
//    128 x 512 tile (1 x 8 wavefronts, same per-wavefront tile):
//    with skewed routing most experts hold a few hundred rows, and padding
//    their tails to 256 rows wasted about a quarter of the MFMA work. The
//    wider tile keeps the weight bytes per MAC unchanged. Both shapes run in
//    one launch from a work list in expert order (groups of 4 M tiles, N tile
//    major inside a group, for L2 reuse), so the weight-bound tiles of
//    experts with few rows overlap the MFMA-bound tiles of the others, and an
//    expert's tail tile finds its weights still cached.
//    The quantised-weight kernels (expert_tile_q.hip) use the 128 x 512 tile
//    throughout (their in-register conversion, not the MFMA, is the bound,
//    and it is done once per column);
//  - K advances 32 per step through four LDS stages filled by direct
//    global->LDS loads (16 B per lane; no registers stage the tiles), issued
//    three steps ahead of the MFMAs, so that a load that misses L2 is hidden
//    by the pipeline depth;
//  - the fragment reads are issued as inline ds_read instructions with
//    explicit waits: the compiler would otherwise wait for every
//    outstanding global->LDS load before any LDS read it can see;
//  - A rows are gathered (token rows of x for gate/up, rows of h for down)
//    and read as K-contiguous 16-byte fragments; B stays in its stored
//    [K, N] layout (N contiguous) and is transposed by ds_read_b64_tr_b16;
//  - every wave instruction that fills LDS writes one contiguous 1 KB
//    block; reads use XOR-swizzled 16-byte granules so the 16 (b128) or 8
//    (transpose) rows read together fall in distinct banks;
//  - for gate/up the tile holds BN/2 gate and the matching BN/2 up columns,
//    so each lane forms silu(gate) * up from two of its own accumulators;
//  - the epilogue goes through LDS so output rows leave in 16-byte stores;
//  - workgroups map onto work items so that consecutive items, which share
//    A rows and B panels, run on the same XCD (and its L2).
#include "tile_common.h"

namespace moe {
namespace {

// One BM x BN output tile (rows m0.. of expert e, N tile nt) of the bf16
// grouped GEMM; smem holds TileShape<WM>::LDS bytes of LDS.
template <bool GATE_UP, int WM, int NW = 4>
__device__ __forceinline__ void tile_bf16_body(const StreamGemmArgs& a, uint8_t* smem, int e,
                                               int m0, int nt) {
  using S = TileShape<WM, NW>;
  constexpr int JT = S::JT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int r0 = a.offsets[e];
  const int cnt = a.offsets[e + 1] - r0;
  const int K = a.K, N = a.N;
  // split-K / weight plane of this workgroup (a single split for the experts)
  const int split = blockIdx.y;
  const int kslice = split % a.nk_split, plane = split / a.nk_split;
  const int lda = a.lda ? a.lda : K;
  const uint16_t* A = a.a + (size_t)kslice * K;
  const uint16_t* W = static_cast<const uint16_t*>(a.w) + (size_t)plane * a.w_plane_stride +
                      (size_t)kslice * K * N;
  float* Yout = a.y_out + (size_t)split * a.y_split_stride;

  // ---- global -> register loads. Rows past the expert's end and columns past
  // N read a clamped valid address: they only feed accumulators never stored.
  // A: instruction q of this wave fills rows ARW*wave + 16q .. +16 (1 KB); lane
  // p holds physical granule p%4 of row ARW*wave + 16q + p/4.
  const uint16_t* asrc[S::QA];
#pragma unroll
  for (int q = 0; q < S::QA; ++q) {
    const int row = S::ARW * wave + 16 * q + (lane >> 2);
    const int lg = (lane & 3) ^ ((row >> 2) & 3);
    size_t grow = 0;
    if (m0 + row < cnt)
      grow = GATE_UP ? (size_t)(a.sorted_pair[r0 + m0 + row] / a.k) : (size_t)(r0 + m0 + row);
    asrc[q] = A + grow * lda + 8 * lg;
  }
  // B: instruction q fills K rows BRW*wave + RPI*q .. +RPI (1 KB); lane p holds
  // physical granule p%(64/RPI) of row BRW*wave + RPI*q + p/(64/RPI).
  const uint16_t* bsrc[S::QB];
  const uint16_t* wbase = W + (size_t)e * K * N;
#pragma unroll
  for (int q = 0; q < S::QB; ++q) {
    const int row = S::BRW * wave + S::RPI * q + lane / (64 / S::RPI);
    const int lg = (lane % (64 / S::RPI)) ^ b_swz(row);
    int col;
    bool ok;
    if (GATE_UP) {
      const int gc = nt * (S::BN / 2) + 8 * (lg % (S::BN / 16));
      ok = gc < a.I;
      col = (lg < S::BN / 16) ? gc : a.I + gc;
    } else {
      col = nt * S::BN + 8 * lg;
      ok = col < N;
    }
    bsrc[q] = wbase + (size_t)row * N + (ok ? col : 0);
  }
  // issue the direct loads of K step kt into stage buffer st
  auto issue = [&](int kt, int st) {
    uint8_t* As = smem + st * S::STAGE;
    uint8_t* Bs = As + S::A_STAGE;
    const int k0 = kt * TBK;
#pragma unroll
    for (int q = 0; q < S::QA; ++q) dma16(asrc[q] + k0, As + (S::ARW * wave + 16 * q) * 64);
#pragma unroll
    for (int q = 0; q < S::QB; ++q)
      dma16(bsrc[q] + (size_t)k0 * N, Bs + (S::BRW * wave + S::RPI * q) * (2 * S::BN));
  };

  f32x16 acc[4][JT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS column of this wave's 32-column tile j (gate/up: JT/2 gate tiles, then
  // the JT/2 matching up tiles)
  auto bcol = [&](int j) -> int {
    constexpr int HW = S::WCOLS / 2, HJ = JT / 2;
    if (GATE_UP) return (j < HJ) ? HW * wn + 32 * j : S::BN / 2 + HW * wn + 32 * (j - HJ);
    return S::WCOLS * wn + 32 * j;
  };
  const int l32 = lane & 31, kh = lane >> 5;  // MFMA row/column and K block
  const int tj = lane & 15, tg = lane >> 4;   // transpose-read lane and group
  const uint32_t lds0 = (uint32_t)(size_t)(lds_u8*)smem;
  // per-lane LDS byte offsets within a stage, for the two 16-deep K halves
  uint32_t aoff[2][4], boff[2][JT][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[s][i] = a_off(128 * wm + 32 * i + l32, 2 * s + kh);
    // B: group tg reads K rows 16s + 8*(tg>>1) + tj/4 (+4) at columns
    // bcol + 16*(tg&1) + 4*(tj%4); the lane receives its column's 8 K values
    const int krow = 16 * s + 8 * (tg >> 1) + (tj >> 2);
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int c = bcol(j) + 16 * (tg & 1) + 4 * (tj & 3);
      boff[s][j][0] = S::A_STAGE + krow * (2 * S::BN) + (((c >> 3) ^ b_swz(krow)) << 4) +
                      ((c & 7) << 1);
      boff[s][j][1] = S::A_STAGE + (krow + 4) * (2 * S::BN) +
                      (((c >> 3) ^ b_swz(krow + 4)) << 4) + ((c & 7) << 1);
    }
  }
  // Fragments of one 16-deep K half: 4 A tiles and JT B tiles (two transpose
  // reads each), 4 + 2 JT reads. Reads are issued asynchronously; the wait
  // macros publish them.
  struct Frag {
    u32x4 a[4];
    u32x2 lo[JT], hi[JT];
  };
  auto read_frag = [&](Frag& f, int st, int s) {
    const uint32_t base = lds0 + st * S::STAGE;
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      f.lo[j] = lds_tr16(base + boff[s][j][0]);
      f.hi[j] = lds_tr16(base + boff[s][j][1]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = lds_b128(base + aoff[s][i]);
  };
  // Wait until at most `pending` LDS reads (those issued after f's) are
  // outstanding; f's registers are operands so nothing consumes them earlier.
#define MOE_LGK_WAIT4(f, pending)                                                             \
  asm volatile("s_waitcnt lgkmcnt(" #pending ")"                                              \
               : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.lo[0]),        \
                 "+v"(f.lo[1]), "+v"(f.lo[2]), "+v"(f.lo[3]), "+v"(f.hi[0]), "+v"(f.hi[1]),   \
                 "+v"(f.hi[2]), "+v"(f.hi[3])                                                  \
               :                                                                               \
               : "memory")
#define MOE_LGK_WAIT2(f, pending)                                                             \
  asm volatile("s_waitcnt lgkmcnt(" #pending ")"                                              \
               : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.lo[0]),        \
                 "+v"(f.lo[1]), "+v"(f.hi[0]), "+v"(f.hi[1])                                   \
               :                                                                               \
               : "memory")
  // wait for f's reads while the next fragment's (4 + 2 JT reads) stay in flight
#define MOE_LGK_WAIT_NEXT(f)   \
  if constexpr (JT == 4)       \
    MOE_LGK_WAIT4(f, 12);      \
  else                         \
    MOE_LGK_WAIT2(f, 8)
#define MOE_LGK_WAIT_ALL(f)    \
  if constexpr (JT == 4)       \
    MOE_LGK_WAIT4(f, 0);       \
  else                         \
    MOE_LGK_WAIT2(f, 0)
  auto mfma_frag = [&](const Frag& f) {
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const u32x4 b = u32x4{f.lo[j][0], f.lo[j][1], f.hi[j][0], f.hi[j][1]};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mfma32(f.a[i], b, acc[i][j]);
    }
  };
  // Pipeline, with a branch-free step body (in-flight fragment registers must
  // never meet a control-flow merge, where copies could read them early):
  // every step issues one K step of loads (clamped to the last step near the
  // end, into the buffer of step kt-1, which is free), so "step kt+1 landed"
  // is always vmcnt(QA + QB); the next half's fragments are always read, the extra
  // read after the last step is discarded. Within a step the second K half's
  // fragments are read while the first half's MFMAs run, and the next step's
  // first half is read (after the barrier that publishes that step's data and
  // frees the buffer of step kt-1) while the second half's MFMAs run.
  const int nk = K / TBK;
  issue(0, 0);
  issue(nk > 1 ? 1 : nk - 1, 1);
  issue(nk > 2 ? 2 : nk - 1, 2);
  // "step kt+1 landed" = at most two later steps (2 * (QA + QB) loads) in flight
  static_assert(S::QA + S::QB == 8 || S::QA + S::QB == 10 || S::QA + S::QB == 4 ||
                    S::QA + S::QB == 5, "vmcnt literals below");
  if constexpr (S::QA + S::QB == 8)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if constexpr (S::QA + S::QB == 10)
    asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
  else if constexpr (S::QA + S::QB == 4)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
  read_frag(f0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    read_frag(f1, kt % NSTAGE, 1);
    MOE_LGK_WAIT_NEXT(f0);
    mfma_frag(f0);
    if constexpr (S::QA + S::QB == 8)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (S::QA + S::QB == 10)
      asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else if constexpr (S::QA + S::QB == 4)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    issue(kt + 3 < nk ? kt + 3 : nk - 1, (kt + 3) % NSTAGE);
    read_frag(f0, (kt + 1) % NSTAGE, 0);
    MOE_LGK_WAIT_NEXT(f1);
    mfma_frag(f1);
  }
  MOE_LGK_WAIT_ALL(f0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef MOE_LGK_WAIT4
#undef MOE_LGK_WAIT2
#undef MOE_LGK_WAIT_NEXT
#undef MOE_LGK_WAIT_ALL
  __builtin_amdgcn_s_barrier();

  // ---- epilogue through LDS (the K loop ended with a barrier, so LDS is free):
  // per 32-row slice the wave writes its results into its own LDS strip, then
  // reads them back row-contiguous for 16-byte global stores. Lane l holds
  // column l%32 of each 32x32 tile at rows 8*(r/4) + 4*(l/32) + r%4.
  auto tile_row = [&](int r) { return 8 * (r >> 2) + 4 * kh + (r & 3); };
  if (GATE_UP) {
    // SW h columns per wavefront (64 or 32), CPR 16-byte chunks per strip row
    constexpr int SW = S::WCOLS / 2, HJ = JT / 2, CPR = SW / 8;
    uint16_t* strip = reinterpret_cast<uint16_t*>(smem + wave * 4096);  // 32 x SW bf16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < HJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          strip[tile_row(r) * SW + 32 * j + l32] =
              (uint16_t)f32_to_bf16_bits(silu(acc[i][j][r]) * acc[i][j + HJ][r]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < SW / 16; ++t) {  // 32 rows x CPR chunks of 16 B
        const int c = lane + 64 * t, rr = c / CPR, ch = c % CPR;
        const int m = m0 + 128 * wm + 32 * i + rr;
        const int col = nt * (S::BN / 2) + SW * wn + 8 * ch;
        const u32x4 v = *reinterpret_cast<const u32x4*>(strip + rr * SW + 8 * ch);
        if (m < cnt && col < a.I)
          *reinterpret_cast<u32x4*>(a.h_out + (size_t)(r0 + m) * a.I + col) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else if (S::WCOLS == 64 && a.y16 != nullptr) {
    // compact rows: this wavefront's strip row is exactly one 64-column scale
    // block; the fp32 results go through LDS as for fp32 rows
    float* strip = reinterpret_cast<float*>(smem + wave * 8192);  // 32 x 64 fp32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) strip[tile_row(r) * 64 + 32 * j + l32] = acc[i][j][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      store_rows16<64>(strip, lane, m0 + 128 * wm + 32 * i, cnt, nt * S::BN + 64 * wn, N,
                       (size_t)r0, a.y16, a.y16_scale);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else {
    constexpr int SW = S::WCOLS, CPR = SW / 4;  // fp32 columns, 16-byte chunks per row
    float* strip = reinterpret_cast<float*>(smem + wave * (32 * SW * 4));  // 32 x SW fp32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) strip[tile_row(r) * SW + 32 * j + l32] = acc[i][j][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < SW / 8; ++t) {  // 32 rows x CPR chunks of 16 B
        const int c = lane + 64 * t, rr = c / CPR, ch = c % CPR;
        const int m = m0 + 128 * wm + 32 * i + rr;
        const int col = nt * S::BN + SW * wn + 4 * ch;
        const f32x4 v = *reinterpret_cast<const f32x4*>(strip + rr * SW + 4 * ch);
        if (m < cnt && col < N) {
          // expert rows stream out; split-K partials of the router are read back at once
          if (a.nsplit == 1)
            store_rows(Yout + (size_t)(r0 + m) * N + col, v);
          else
            *reinterpret_cast<f32x4*>(Yout + (size_t)(r0 + m) * N + col) = v;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}


// Work item -> workgroup: consecutive items (same M tile, neighbouring N
// tiles) run on one XCD, whose L2 they share. Workgroups are dealt to the
// eight XCDs round robin, so XCD x takes items [x * per, (x + 1) * per).
__device__ __forceinline__ int xcd_item(int total) {
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = (total + 7) >> 3;
  if (slot >= per) return -1;
  const int w = xcd * per + slot;
  return w < total ? w : -1;
}

// One tile shape: M-tile table x NT N tiles.
template <bool GATE_UP, int WM>
__global__ __launch_bounds__(256, 1) void tile_bf16_kernel(StreamGemmArgs a,
                                                           const int32_t* __restrict__ tile_e,
                                                           const int32_t* __restrict__ tile_m0,
                                                           const int32_t* __restrict__ n_tiles_p,
                                                           int NT) {
  __shared__ __align__(1024) uint8_t smem[TileShape<WM>::LDS];
  const int w = xcd_item(*n_tiles_p * NT);
  if (w < 0) return;
  const int mt = w / NT, nt = w - mt * NT;
  tile_bf16_body<GATE_UP, WM>(a, smem, tile_e[mt], tile_m0[mt], nt);
}

// Both tile shapes in one launch, from a work list in expert order (each
// expert's 256-row tiles, then its last <= 128 rows as a 128 x 512 tile):
// an expert's tiles run close together, while its weights are still cached,
// and the HBM-bound tiles of experts with few rows overlap the MFMA-bound
// tiles of the others instead of running after them. Item: x = e | kind << 8
// | nt << 9 (kind 1: 128 x 512 tile), y = first row.
template <bool GATE_UP, int NW>
__global__ __launch_bounds__(64 * NW, 1) void tile_bf16_mixed_kernel(StreamGemmArgs a,
                                                                     const int2* __restrict__ items,
                                                                     const int32_t* __restrict__ n_items_p) {
  static_assert(TileShape<1>::LDS >= TileShape<2>::LDS, "LDS sized for the larger tile");
  __shared__ __align__(1024) uint8_t smem[TileShape<1>::LDS];
  const int w = xcd_item(*n_items_p);
  if (w < 0) return;
  const int2 it = items[w];
  const int e = it.x & 0xff, nt = it.x >> 9;
  if (it.x & 0x100)
    tile_bf16_body<GATE_UP, 1, NW>(a, smem, e, it.y, nt);
  else
    tile_bf16_body<GATE_UP, 2, NW>(a, smem, e, it.y, nt);
}

#ifndef MOE_TILE_GM
#define MOE_TILE_GM 4
#endif
// Work lists of the mixed launch, one per blockIdx.y (gate/up, down). Expert e
// with c rows has c / 256 full tiles, plus one more if c % 256 > 128, else one
// 128-row tile if c % 256 > 0; a full tile spans ntf N tiles, a 128-row tile
// nth. Every workgroup rebuilds the per-expert scan and writes the items
// blockIdx.x * 256 .. +255 of the list.
__global__ __launch_bounds__(256) void tile_items_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int ntf0, int nth0, int2* __restrict__ items0,
                                                         int32_t* __restrict__ n0, int ntf1, int nth1,
                                                         int2* __restrict__ items1,
                                                         int32_t* __restrict__ n1) {
  __shared__ int incl[256], nfull[256];
  const int g = blockIdx.y;
  const int ntf = g ? ntf1 : ntf0, nth = g ? nth1 : nth0;
  int2* items = g ? items1 : items0;
  const int e = threadIdx.x;
  const int rows = (e < E) ? offsets[e + 1] - offsets[e] : 0;
  const int rem = rows & 255;
  const int half = (rem > 0 && rem <= 128) ? 1 : 0;
  const int full = (rows >> 8) + (rem > 128 ? 1 : 0);
  const int mine = full * ntf + half * nth;
  incl[e] = mine;
  nfull[e] = full;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {  // inclusive scan
    const int v = (e >= d) ? incl[e - d] : 0;
    __syncthreads();
    incl[e] += v;
    __syncthreads();
  }
  const int total = incl[255];
  if (blockIdx.x == 0 && e == 0) *(g ? n1 : n0) = total;
  const int w = blockIdx.x * 256 + e;
  if (w >= total) return;
  int lo = 0, hi = 255;  // the expert: smallest x with incl[x] > w
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (incl[mid] > w)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int x = lo;
  const int local = w - (x ? incl[x - 1] : 0);
  const int fcount = nfull[x] * ntf;
  int2 it;
  if (local < fcount) {
    // groups of GM full M tiles; inside a group N tile major, so the items
    // one XCD runs at a time span GM M tiles and a few N tiles
    const int grp = local / (MOE_TILE_GM * ntf), in = local - grp * (MOE_TILE_GM * ntf);
    const int rest = nfull[x] - grp * MOE_TILE_GM;
    const int gm = rest < MOE_TILE_GM ? rest : MOE_TILE_GM;
    const int ntile = in / gm, mt = grp * MOE_TILE_GM + (in - ntile * gm);
    it.x = x | (ntile << 9);
    it.y = mt * 256;
  } else {
    it.x = x | 0x100 | ((local - fcount) << 9);
    it.y = nfull[x] * 256;
  }
  items[w] = it;
}

// fp32 router weights [H, E] -> three bf16 planes [3][H][256] (columns >= E zero):
// hi = RNE(w), mid = RNE(w - hi), lo = RNE(w - hi - mid); both differences are
// exact in fp32. Also writes the one-expert offsets {0, T} the tiled kernel uses.
__global__ __launch_bounds__(256) void router_pack_kernel(const float* __restrict__ w, int H, int E,
                                                          uint16_t* __restrict__ planes,
                                                          int32_t* __restrict__ offsets, int T) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // over H * 256
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
  }
  if (i >= (size_t)H * 256) return;
  const int h = (int)(i >> 8), c = (int)(i & 255);
  const float v = c < E ? w[(size_t)h * E + c] : 0.f;
  const uint32_t hi = f32_to_bf16_bits(v);
  const float r1 = v - bf16_bits_to_f32(hi);
  const uint32_t mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(mid);
  const uint32_t lo = f32_to_bf16_bits(r2);
  const size_t plane = (size_t)H * 256;
  planes[i] = (uint16_t)hi;
  planes[plane + i] = (uint16_t)mid;
  planes[2 * plane + i] = (uint16_t)lo;
}

constexpr int ROUTER_NKS = 2;  // K slices per plane (3 * 2 splits in all)

// Wavefronts per workgroup of the mixed launch: 8 (128 x 64 each, two per
// SIMD). The compact-row epilogue needs each wavefront's strip to be one
// 64-column scale block.
constexpr int kMixedWaves = 8;
static_assert(TileShape<2, kMixedWaves>::WCOLS == 64 && TileShape<1, kMixedWaves>::WCOLS == 64,
              "compact rows take one 64-column block per wavefront strip");

// Tile counts of the mixed launch: N tiles of a full (256 x 256) tile and of a
// 128-row (128 x 512) tile, and the largest work list.
struct MixedPlan {
  int ntf, nth, max_items;
};
MixedPlan mixed_plan(bool gate_up, int P, int E, int N, int I) {
  MixedPlan m;
  m.ntf = gate_up ? (I + 127) / 128 : (N + 255) / 256;
  m.nth = gate_up ? (I + 255) / 256 : (N + 511) / 512;
  m.max_items = ((P + TBM - 1) / TBM + E) * m.ntf + E * m.nth;
  return m;
}

}  // namespace

bool expert_tile_fits(long long P, int E, int H, int I) {
  // the work lists of the mixed launches are indexed with int
  const long long full = (P + TBM - 1) / TBM + E;
  const long long g = full * ((I + 127) / 128) + (long long)E * ((I + 255) / 256);
  const long long d = full * (((long long)H + 255) / 256) + (long long)E * (((long long)H + 511) / 512);
  return g < (1LL << 30) && d < (1LL << 30);
}

size_t expert_tile_ws_bytes(int P, int E, int H, int I) {
  // the larger of: the table of 128-row tiles (quantised weights), and the
  // counters plus the two work lists of the mixed bf16 launches
  const int max_tiles = (P + 127) / 128 + E;
  const size_t q = (size_t)(2 * max_tiles + 64) * sizeof(int32_t);
  const size_t b = 256 + ((size_t)mixed_plan(true, P, E, 2 * I, I).max_items +
                          mixed_plan(false, P, E, H, I).max_items) * sizeof(int2);
  return q > b ? q : b;
}

int router_bf16x3_splits() { return 3 * ROUTER_NKS; }

size_t router_bf16x3_ws_bytes(int T, int H) {
  const int tiles = (T + TBM - 1) / TBM + 1;
  return (size_t)3 * H * 256 * sizeof(uint16_t) + (size_t)(2 * tiles + 64) * sizeof(int32_t) + 256;
}

hipError_t launch_router_bf16x3(const uint16_t* x, int T, int H, const float* w_router, int E,
                                float* part, void* ws, hipStream_t st) {
  if (H % (TBK * ROUTER_NKS) != 0) return hipErrorInvalidValue;
  uint16_t* planes = static_cast<uint16_t*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(planes + (size_t)3 * H * 256);
  const int max_tiles = (T + TBM - 1) / TBM + 1;
  int32_t* tile_e = offsets + 64;
  int32_t* tile_m0 = tile_e + max_tiles;
  int32_t* n_tiles = tile_m0 + max_tiles;
  router_pack_kernel<<<(unsigned)(((size_t)H * 256 + 255) / 256), 256, 0, st>>>(w_router, H, E, planes,
                                                                              offsets, T);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  tile_table_kernel<<<1, 256, 0, st>>>(offsets, 1, TBM, 0, tile_e, tile_m0, n_tiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  StreamGemmArgs a{};
  a.a = x;
  a.offsets = offsets;
  a.sorted_pair = nullptr;
  a.k = 1;
  a.E = 1;
  a.K = H / ROUTER_NKS;
  a.lda = H;
  a.N = 256;
  a.I = 0;
  a.w = planes;
  a.y_out = part;
  a.nsplit = 3 * ROUTER_NKS;
  a.nk_split = ROUTER_NKS;
  a.w_plane_stride = (long long)H * 256;
  a.y_split_stride = (long long)T * 256;
  const unsigned grid = (unsigned)(((max_tiles + 7) / 8) * 8);
  tile_bf16_kernel<false, 2><<<dim3(grid, a.nsplit), 256, 0, st>>>(a, tile_e, tile_m0, n_tiles, 1);
  return hipGetLastError();
}

static hipError_t launch_bf16_all(const StreamGemmArgs& gu, const StreamGemmArgs& dn, int P,
                                  int2* items_g, int2* items_d, int32_t* counts, hipStream_t st) {
  const MixedPlan pg = mixed_plan(true, P, gu.E, gu.N, gu.I);
  const MixedPlan pd = mixed_plan(false, P, dn.E, dn.N, dn.I);
  const int most = pg.max_items > pd.max_items ? pg.max_items : pd.max_items;
  tile_items_kernel<<<dim3((unsigned)((most + 255) / 256), 2), 256, 0, st>>>(
      gu.offsets, gu.E, pg.ntf, pg.nth, items_g, counts, pd.ntf, pd.nth, items_d, counts + 1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  tile_bf16_mixed_kernel<true, kMixedWaves><<<(unsigned)((pg.max_items + 7) / 8 * 8),
                                               64 * kMixedWaves, 0, st>>>(gu, items_g, counts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  tile_bf16_mixed_kernel<false, kMixedWaves><<<(unsigned)((pd.max_items + 7) / 8 * 8),
                                                64 * kMixedWaves, 0, st>>>(dn, items_d, counts + 1);
  return hipGetLastError();
}

// Quantised weights run on 128 x 512 tiles only. Their wavefronts sit side by
// side along N, so each B column is converted by one wavefront (in the 2 x 2
// layout of the 256 x 256 tile two wavefronts convert every column, and the
// conversion is what bounds these kernels).
hipError_t launch_expert_tile(int wfmt, const StreamGemmArgs& gu, const StreamGemmArgs& dn, int P,
                              void* ws, hipStream_t st) {
  const int E = gu.E;
  int32_t* tile_e = static_cast<int32_t*>(ws);
  if (wfmt == W_FP8 || wfmt == W_FP4) return launch_expert_tile_q(wfmt, gu, dn, P, ws, st);
  if (wfmt != W_BF16) return hipErrorInvalidValue;
  // work lists of the mixed 256 x 256 / 128 x 512 launches
  const MixedPlan pg = mixed_plan(true, P, E, gu.N, gu.I);
  int32_t* counts = tile_e;  // [0]: gate/up items, [1]: down items
  int2* items_g = reinterpret_cast<int2*>(static_cast<char*>(ws) + 256);
  int2* items_d = items_g + pg.max_items;
  return launch_bf16_all(gu, dn, P, items_g, items_d, counts, st);
}

}  // namespace moe
