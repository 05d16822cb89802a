// Grouped SwiGLU expert GEMMs with FP8 (E4M3, per-channel scales) and NVFP4
// (E2M1 codes, E4M3 scale per 16 values, fp32 scale per expert) weights for
// few rows per expert (decode-sized batches), on gfx950 MFMA, in the mode
// that dequantises the weights exactly (bf16 activations; the pages' NVFP4
// variant runs with BF16 activations: vLLM recipe
// "reflection/Beam-1.0-501B-A23B", Guide > Variants). Work split, grid and
// split-K partial sums are those of the bf16 streaming kernels
// (expert_stream.hip); the weights are stored [N, K] (K contiguous).
#include <type_traits>

#include "stream_common.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ FP8 weights
// K-contiguous E4M3 weights [E, N, K] with one fp32 scale per output channel.
// Per "super step" the four lane groups of a column each read 32 B of it,
// together one whole 128 B line (32 K values per lane). (Reading half a line
// per super step measured 2.8x the algorithmic bytes fetched at decode:
// lines were evicted before their second half was used; and the default
// cache policy measured 1.3x faster than nontemporal loads here.)
// A workgroup's four wavefronts own 64 columns each of the same expert and K
// range, so the A rows of a super step (x or h, 8 KB) are loaded once into
// LDS by direct buffer -> LDS loads (each wavefront a quarter) and shared;
// the weight codes go to registers (buffer loads with the expert's matrix as
// the buffer), three super steps rotating through three register sets, so
// two super steps of loads are in flight while one is converted. Every
// wavefront issues the same loads per super step (idle ones read column tile
// 0 and store nothing), so "A of step ss landed" is one vmcnt for all. Codes
// become bf16 exactly with the hardware converter; the per-channel scales
// multiply the accumulators. In MFMA s of a super step lane group g covers
// K ss*SPAN + G*g + 8s .. +8, for A and B alike.
#ifndef MOE_KM_CPOL
#define MOE_KM_CPOL 0  // cache policy of the code loads (0: default, 2: nontemporal)
#endif
template <int WF>
struct KmShape {
  static_assert(WF == W_FP8, "E4M3 weights");
  static constexpr int G = 32;                       // K values per lane per super step
  static constexpr int NS = G / 8;                   // MFMA K steps per super step
  static constexpr int SPAN = 4 * G;                 // K per super step
  static constexpr int NV = 2;                       // 16 B code loads per lane and column
  static constexpr int CG = 4;                       // 16-column groups per wavefront
  static constexpr int COLS = 16 * CG;               // columns per wavefront
  static constexpr int NF = 2;                       // 16-row fragments per pass
  static constexpr int AROWS = 16 * NF;              // A rows per pass
  static constexpr int AROWB = SPAN * 2;             // bytes of an A row per super step
  static constexpr int ACH = AROWB / 16;             // 16 B chunks per A row
  static constexpr int ASLOT = AROWS * AROWB;        // LDS bytes of A per super step
  static constexpr int NSLOT = 3;                    // super steps of A in LDS
  static constexpr int RPI = 1024 / AROWB;           // A rows per 1 KB direct load
  static constexpr int DPW = ASLOT / 1024 / 4;       // direct loads per wavefront per super step
  static constexpr int NWL = CG * NV;                // weight loads per super step
  static_assert(DPW * 4 * 1024 == ASLOT && AROWS % (4 * DPW) == 0, "A tile split");
};

// Direct buffer -> LDS load: lane l's 16 bytes (at byte offset off of the
// buffer) land at lds + 16 * l. The buffer form keeps the compiler's own
// vmcnt waits for the register loads beside it exact (a FLAT-encoded
// load to LDS counts as possibly pending on both counters, after which the
// compiler waits for everything).
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0,
                                           0, 0);
}
// LDS read the compiler does not see (valid after an explicit lgkmcnt wait
// that takes it as an operand).
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

template <int WF, bool GATE_UP>
__global__ __launch_bounds__(256, 2) void stream_kmajor_kernel(StreamGemmArgs a) {
  using S = KmShape<WF>;
  constexpr int G = S::G, NS = S::NS, SPAN = S::SPAN, NV = S::NV, CG = S::CG, NF = S::NF;
  __shared__ __align__(16) uint8_t als[S::NSLOT * S::ASLOT];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int tile = blockIdx.x * 4 + wave;
  const int n_tiles = GATE_UP ? a.I / (S::COLS / 2) : (a.N + S::COLS - 1) / S::COLS;
  const bool tile_ok = tile < n_tiles;  // idle wavefronts still load A and meet the barriers
  // expert, rows and K range: the same for the whole workgroup
  const int e = slot_expert(a.offsets, a.E, blockIdx.y, lane);
  if (e < 0) return;
  const int r0 = a.offsets[e];
  const int cnt = a.offsets[e + 1] - r0;
  if (cnt <= 0) return;
  const int K = a.K, N = a.N;
  const int nss = (K + SPAN - 1) / SPAN;
  const int split = blockIdx.z;
  const int ss0 = a.ksplit > 1 ? split * a.ksteps : 0;
  const int ss1 = a.ksplit > 1 ? min(nss, ss0 + a.ksteps) : nss;
  if (ss0 >= ss1) return;

  // this lane's CG columns (gate/up: CG/2 gate, then the matching up columns);
  // columns past N read column 0 and are never stored
  const int row_bytes = K;
  // this expert's codes as a buffer (31-bit size, checked by the host)
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const uint8_t*>(a.w) + (size_t)e * N * row_bytes), (short)0, N * row_bytes,
      0x00020000);
  const int tc = tile_ok ? tile : 0;
  int colv[CG];
  bool cok[CG];
  uint32_t coff[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    constexpr int H2 = CG / 2, HC = S::COLS / 2;
    if (GATE_UP)
      colv[cg] = cg < H2 ? tc * HC + 16 * cg + j : a.I + tc * HC + 16 * (cg - H2) + j;
    else
      colv[cg] = tc * S::COLS + 16 * cg + j;
    cok[cg] = tile_ok && colv[cg] < N;
    coff[cg] = (uint32_t)(colv[cg] < N ? colv[cg] : 0);
  }
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)als;
  auto clampss = [&](int x) { return x < ss1 ? x : ss1 - 1; };
  // A as a buffer: x ([rows / k, K]) for gate/up, h ([rows, K]) for down; its
  // byte size fits 31 bits (checked by the host)
  const uint32_t a_bytes = (uint32_t)((GATE_UP ? a.rows / a.k : a.rows) * (long long)K * 2);
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.a, (short)0, (int)a_bytes, 0x00020000);

  for (int mc = 0; mc < cnt; mc += S::AROWS) {
    const int nf = (NF == 2 && (cnt - mc) > 16) ? 2 : 1;
    // A rows this wavefront loads: direct load d covers rows RPI * (DPW * wave + d) ..
    // (lane / ACH within), 16 B chunk position lane % ACH holding K chunk
    // (lane % ACH) ^ (row % ACH) (the XOR keeps the 16 rows a fragment read
    // touches in distinct banks)
    uint32_t arow[S::DPW];  // element offsets of the rows in A
    int achk[S::DPW];
#pragma unroll
    for (int d = 0; d < S::DPW; ++d) {
      const int row = S::RPI * (S::DPW * wave + d) + lane / S::ACH;
      const int m = mc + row;
      uint32_t grow = 0;
      if (m < cnt) grow = GATE_UP ? (uint32_t)(a.sorted_pair[r0 + m] / a.k) : (uint32_t)(r0 + m);
      arow[d] = grow * (uint32_t)K;
      achk[d] = 8 * ((lane % S::ACH) ^ (row % S::ACH));
    }
    auto issue_a = [&](int ss, int slot) {
#pragma unroll
      for (int d = 0; d < S::DPW; ++d) {
        // chunks past K (a K tail) read the row's first chunk; their products are zeroed
        const int ko = ss * SPAN + achk[d];
        dma16s(arsrc, 2u * (arow[d] + (uint32_t)(ko < K ? ko : 0)),
               als + slot * S::ASLOT + S::RPI * (S::DPW * wave + d) * S::AROWB);
      }
    };
    f32x4 acc[NF][CG];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < CG; ++i) acc[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct Ops {
      u32x4 b[CG][NV];
    };
    auto load_ops = [&](int ss, Ops& o) {
      const int kl = ss * SPAN + G * g;
      const uint32_t kc = kl < K ? (uint32_t)kl : 0u;
#pragma unroll
      for (int cg = 0; cg < CG; ++cg)
#pragma unroll
        for (int v = 0; v < NV; ++v)
          o.b[cg][v] =
              __builtin_amdgcn_raw_buffer_load_b128(wrsrc, coff[cg] * (uint32_t)row_bytes + kc + 16 * v, 0, MOE_KM_CPOL);
    };
    // one super step: wait for its loads (only step ss + 1's may still be in
    // flight, whatever order the loads of a step were issued in; the barrier
    // publishes the other wavefronts' A and frees the slot of step ss - 1),
    // issue step ss + 2, read the A fragments, convert and multiply
    auto step = [&](int ss, Ops& cur, Ops& next2) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(S::NWL + S::DPW) : "memory");
      __builtin_amdgcn_s_barrier();
      issue_a(clampss(ss + 2), (ss + 2) % S::NSLOT);
      load_ops(clampss(ss + 2), next2);
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t slot = lds_base + (ss % S::NSLOT) * S::ASLOT;
      static_assert(NF * NS == 8, "eight A fragments per super step");
      u32x4 af[8];
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          const int row = 16 * f + j;
          const int ch = ((G * g + 8 * q) / 8) ^ (row % S::ACH);
          af[NS * f + q] = lds_read16(slot + row * S::AROWB + 16 * ch);
        }
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(af[4]), "+v"(af[5]),
                     "+v"(af[6]), "+v"(af[7])
                   :
                   : "memory");
      const bool kok = ss * SPAN + G * g < K;  // false only in a K tail
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          const u32x4 bf = fp8_frag(cur.b[cg][q >> 1][2 * (q & 1)], cur.b[cg][q >> 1][2 * (q & 1) + 1]);
#pragma unroll
          for (int f = 0; f < NF; ++f)
            if (f < nf) acc[f][cg] = mfma_bf16(kok ? af[NS * f + q] : zero, bf, acc[f][cg]);
        }
        // one column group at a time: converting ahead would need registers
        // the third weight set holds
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // the previous pass's LDS reads and direct loads are done before the
    // slots are refilled
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    Ops w0, w1, w2;
    issue_a(ss0, ss0 % S::NSLOT);
    load_ops(ss0, w0);
    issue_a(clampss(ss0 + 1), (ss0 + 1) % S::NSLOT);
    load_ops(clampss(ss0 + 1), w1);
    int ss = ss0;
    for (; ss + 2 < ss1; ss += 3) {
      step(ss, w0, w2);
      step(ss + 1, w1, w0);
      step(ss + 2, w2, w1);
    }
    if (ss < ss1) step(ss, w0, w2);  // w0 holds step ss, w1 step ss + 1
    if (ss + 1 < ss1) step(ss + 1, w1, w0);

    // epilogue: lane (g, j) holds rows 16f + 4g + r of column colv[cg]
    const float* chs = static_cast<const float*>(a.w_scale) + (size_t)e * N;
    float csc[CG];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) csc[cg] = chs[coff[cg]];
    float* pbase = a.ksplit > 1 ? a.part + (size_t)split * a.part_stride : nullptr;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f >= nf) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mc + 16 * f + 4 * g + r;
        if (m >= cnt || !tile_ok) continue;
        if (pbase) {  // split K: scaled fp32 partial sums
#pragma unroll
          for (int cg = 0; cg < CG; ++cg)
            if (cok[cg]) pbase[(size_t)(r0 + m) * N + colv[cg]] = acc[f][cg][r] * csc[cg];
        } else if (GATE_UP) {
#pragma unroll
          for (int cg = 0; cg < CG / 2; ++cg) {
            const float gv = acc[f][cg][r] * csc[cg], uv = acc[f][cg + CG / 2][r] * csc[cg + CG / 2];
            a.h_out[(size_t)(r0 + m) * a.I + colv[cg]] = (uint16_t)f32_to_bf16_bits(silu(gv) * uv);
          }
        } else {
#pragma unroll
          for (int cg = 0; cg < CG; ++cg)
            if (cok[cg]) store_rows(a.y_out + (size_t)(r0 + m) * N + colv[cg], acc[f][cg][r] * csc[cg]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ NVFP4 weights
// E2M1 codes [E, N, K/2] with one E4M3 scale per 16 K values.
// The block scale is not multiplied into the weights. Since w = e2m1 * s,
// sum_k x_k w_k = sum over blocks of s * (sum over the block of x_k e2m1_k):
// the codes become bf16 with the hardware converter at scale 1 (exact), a
// 4x4x4 MFMA chain forms each 16-value block's partial sums on their own, and
// one fp32 FMA per output applies the block scale (its exact fp32 value). At
// up to four rows per MFMA that is a quarter of an FMA per weight value
// instead of a multiply per value.
// Memory: a wavefront owns 32 columns (4 groups of 8) of one expert's matrix;
// per super step (256 K values) each of its load instructions reads whole
// 128 B lines, 8 lanes x 16 B per column for 8 columns (measured with the
// same access pattern: 5.9 TB/s, against 4.4 TB/s for 4 lanes x 2 x 16 B per
// line plus a scale dword per lane and step). The block scales of 8 super
// steps (128 B per column) reach LDS by direct loads of whole lines, half a
// wavefront's worth per super step, two blocks of 8 steps ahead; the A rows
// (x or h) of a super step are loaded once per workgroup into LDS (each
// wavefront a quarter) and shared; codes go to registers, super steps rotating
// through NSET register sets. Loads use the default cache policy (measured
// faster than nontemporal for this pattern). A workgroup whose K range is at
// most one scale block (the down GEMM at the decode shape: 6 super steps)
// instead loads the A rows of all its steps and its scale block once per pass:
// its K loop then issues only code loads and meets no barrier (measured: the
// per-step direct loads and barrier cost that kernel 17%).
// MFMA v_mfma_f32_4x4x4_16b_bf16 (16 independent 4x4 blocks, K = 4): lane l
// belongs to block l/4, supplies A row l%4 and B column l%4 (4 K values
// each), and its result holds column l%4 of its block for rows 0..3. Here
// lane l's block is (K range q = l/8, column half (l/4)%2): the lane works on
// column 8 cg + l%8 over K range q (32 values of each super step), with rows
// (tokens) 4 rg + l%4 as A. After the K loop the eight K ranges' partial
// sums are added across lanes l, l^8, l^16, l^32.
#ifndef MOE_FP4_NSET
#define MOE_FP4_NSET 2  // code register sets at up to 8 rows per pass
#endif
#ifndef MOE_FP4_CHAINS
#define MOE_FP4_CHAINS 4  // independent MFMA chains in flight
#endif
template <int RG>
struct Fp4Shape {
  static constexpr int KQ = 8;                   // K ranges of a super step (lanes / 8)
  static constexpr int G = 32;                   // K values per lane per super step
  static constexpr int SPAN = KQ * G;            // K per super step
  static constexpr int CG = 4;                   // 8-column groups per wavefront
  static constexpr int COLS = 8 * CG;            // columns per wavefront
  static constexpr int AROWS = 4 * RG;           // A rows per pass (RG row groups of 4)
  static constexpr int AROWB = SPAN * 2;         // bytes of an A row per super step
  static constexpr int ACH = AROWB / 16;         // 16 B chunks per A row
  static constexpr int ASLOT = AROWS * AROWB;    // LDS bytes of A per super step
  static constexpr int NSLOT = 4;                // super steps of A in LDS (at least the code sets)
  static constexpr int RPI = 1024 / AROWB;       // A rows per 1 KB direct load
  static constexpr int DPW = ASLOT / 1024 / 4;   // direct A loads per wavefront per super step
  static constexpr int SBLK = 8;                 // super steps per scale block
  static constexpr int SSLOT = COLS * SBLK * 16;  // scale bytes of a wavefront per block
  static constexpr int NWL = CG + 1;             // loads per super step: codes + half a scale block piece
  static_assert(DPW >= 1 && DPW * 4 * 1024 == ASLOT, "A tile split");
  static_assert(SSLOT == SBLK * 512, "one half-wavefront scale load per super step");
};

// LDS position of 16 B K chunk c (0..31) of A row t, XOR-swizzled so that the
// chunks one fragment read touches (4 rows x 8 K ranges) spread over the
// banks. An involution: it maps positions back to chunks too.
__device__ __forceinline__ int fp4_apos(int c, int t) { return c ^ (t & 3) ^ (((c >> 4) & 1) << 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 4 E2M1 codes (bytes SEL, SEL + 1 of d) -> 4 bf16 (exact)
template <int SEL>
__device__ __forceinline__ u32x2 e2m1_bf16_4(uint32_t d) {
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, SEL)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, SEL + 1))};
}
// 4x4x4 MFMA on half AH (regs 2 AH, 2 AH + 1) of A and a 2-register B
template <int AH>
__device__ __forceinline__ f32x4 mfma4h(const u32x4& a, const u32x2& b, const f32x4& c) {
  const u32x2 av = {a[2 * AH], a[2 * AH + 1]};
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, av), __builtin_bit_cast(s16x4, b),
                                                c, 0, 0, 0);
}
// LDS reads the compiler does not see (valid after an explicit lgkmcnt wait
// that takes them as operands), at addr + OFF
template <int OFF>
__device__ __forceinline__ uint32_t lds_read_u16o(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16o(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}

// KT: K has a tail (K % SPAN != 0), whose chunks are clamped and whose block
// scales are zeroed; without one those checks compile away.
template <int RG, bool GATE_UP, bool KT, bool AR>
__global__ __launch_bounds__(256, 2) void stream_fp4_kernel(StreamGemmArgs a) {
  using S = Fp4Shape<RG>;
  static_assert(RG == 2, "8 rows per pass: 16 need more registers than two workgroups per CU allow");
  constexpr int SPAN = S::SPAN, CG = S::CG;
  // AR (the K range is at most one scale block, SBLK super steps): the A rows
  // of every step and the wavefront's scale block are loaded once per pass and
  // stay in LDS, so the K loop issues only its code loads and needs no
  // barrier. Otherwise A and the scales stream through rings refilled per step.
  constexpr int ASL = AR ? S::SBLK : S::NSLOT;  // A slots
  constexpr int NSB = AR ? 1 : 3;               // scale blocks per wavefront
  __shared__ __align__(16) uint8_t als[ASL * S::ASLOT];
  __shared__ __align__(16) uint8_t sls[4][NSB * S::SSLOT];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane >> 3, c8 = lane & 7;  // K range, column within an 8-column group
  const int tile = blockIdx.x * 4 + wave;
  const int n_tiles = GATE_UP ? a.I / (S::COLS / 2) : (a.N + S::COLS - 1) / S::COLS;
  const bool tile_ok = tile < n_tiles;  // idle wavefronts still load and meet the barriers
  // expert, rows and K range: the same for the whole workgroup
  const int e = slot_expert(a.offsets, a.E, blockIdx.y, lane);
  if (e < 0) return;
  const int r0 = a.offsets[e];
  const int cnt = a.offsets[e + 1] - r0;
  if (cnt <= 0) return;
  const int K = a.K, N = a.N;
  const int nss = (K + SPAN - 1) / SPAN;
  const int split = blockIdx.z;
  const int ss0 = a.ksplit > 1 ? split * a.ksteps : 0;
  const int ss1 = a.ksplit > 1 ? min(nss, ss0 + a.ksteps) : nss;
  if (ss0 >= ss1) return;

  // this expert's codes and block scales as buffers (31-bit sizes, checked by the host)
  const int row_bytes = K / 2, srow = K / 16;
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const uint8_t*>(a.w) + (size_t)e * N * row_bytes), (short)0, N * row_bytes,
      0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const uint8_t*>(a.w_scale) + (size_t)e * N * srow), (short)0, N * srow,
      0x00020000);
  // this lane's CG columns (gate/up: CG/2 gate groups, then the matching up
  // groups); columns past N read column 0 and are never stored
  const int tc = tile_ok ? tile : 0;
  auto column = [&](int cg, int c) {
    constexpr int H2 = CG / 2, HC = S::COLS / 2;
    if (GATE_UP) return cg < H2 ? tc * HC + 8 * cg + c : a.I + tc * HC + 8 * (cg - H2) + c;
    return tc * S::COLS + 8 * cg + c;
  };
  uint32_t coff[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const int col = column(cg, c8);
    coff[cg] = (uint32_t)(col < N ? col : 0) * (uint32_t)row_bytes;
  }
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)als;
  uint8_t* const swave = sls[wave];
  const uint32_t sbase = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)swave;
  auto clampss = [&](int x) { return x < ss1 ? x : ss1 - 1; };
  // A as a buffer: x ([rows / k, K]) for gate/up, h ([rows, K]) for down
  const uint32_t a_bytes = (uint32_t)((GATE_UP ? a.rows / a.k : a.rows) * (long long)K * 2);
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.a, (short)0, (int)a_bytes, 0x00020000);
  // LDS byte offsets (within a slot) of this lane's A chunks: row lane % 4 (+ 4 rg),
  // K chunk 4 q + h (h: 16 B piece of the lane's 64 B)
  uint32_t aoff[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) aoff[h] = (uint32_t)((lane & 3) * S::AROWB + 16 * fp4_apos(4 * q + h, lane & 3));
  // block scales in the wavefront's LDS: column cw = 8 cg + c8 at cw * 128, step
  // st of the block at + 16 st, blocks 2q, 2q + 1 at + 2q
  const uint32_t scoff = (uint32_t)(c8 * 128 + 2 * q);
  // half-wavefront scale load st of scale block rb (super steps ss0 + 8 rb ..):
  // lane l < 32 reads chunk l % 8 (one super step) of column 4 st + l / 8 of
  // this wavefront's 32
  auto issue_s = [&](int rb, int st) {
    const int cw = 4 * st + (lane >> 3) % 4;
    const int col = column(cw >> 3, cw & 7);
    const int k16 = (ss0 + S::SBLK * rb) * (SPAN / 16) + 16 * (lane & 7);  // scale byte of this chunk
    const uint32_t off = (uint32_t)(col < N ? col : 0) * (uint32_t)srow + (uint32_t)(k16 + 16 <= srow ? k16 : 0);
    if (lane < 32) dma16s(srsrc, off, swave + (rb % NSB) * S::SSLOT + st * 512);
  };

  // One pass over K for rows mc .. mc + 4 NRG - 1 (NRG row groups; padding
  // rows are computed and not stored). The row-group count is a compile-time
  // constant: branching on it inside the K loop costs registers.
  auto pass = [&](int mc, auto nrg_c) {
    constexpr int NRG = decltype(nrg_c)::value;
    static_assert(NRG == 1 || NRG == 2, "one or two row groups");
    // (the down GEMM's short K range, 6 super steps at the decode shape,
    // gains from a third code set at up to 4 rows: 4% on that kernel)
    constexpr int NSET = (!GATE_UP && NRG == 1) ? 3 : MOE_FP4_NSET;
    static_assert(NSET <= S::NSLOT, "A slots for every step in flight");
    // column groups whose MFMA chains run side by side
    constexpr int CI = (MOE_FP4_CHAINS / NRG) < 1 ? 1 : (MOE_FP4_CHAINS / NRG) > CG ? CG : MOE_FP4_CHAINS / NRG;
    // A rows this wavefront loads: direct load d covers rows RPI * (DPW * wave + d)
    // (+ lane / ACH), position lane % ACH holding K chunk fp4_apos(lane % ACH, row)
    uint32_t arow[S::DPW];
    int achk[S::DPW];
#pragma unroll
    for (int d = 0; d < S::DPW; ++d) {
      const int row = S::RPI * (S::DPW * wave + d) + lane / S::ACH;
      const int m = mc + row;
      uint32_t grow = 0;
      if (m < cnt) grow = GATE_UP ? (uint32_t)(a.sorted_pair[r0 + m] / a.k) : (uint32_t)(r0 + m);
      arow[d] = grow * (uint32_t)K;
      achk[d] = 8 * fp4_apos(lane % S::ACH, row);
    }
    // all loads of super step ss, issued while step ss - NSET + 1 runs: A
    // rows, this lane's codes, and (uniformly, one per issue) a half-wavefront
    // piece of scale block b + 2, b being the running step's block. A block's
    // pieces are issued in the 8 steps after the block three before it (same
    // LDS slot) was last read; the issues before the first step repeat pieces
    // of block 1 (same data, slot not yet read).
    // (measured: handing the step's K offset to the loads as their scalar
    // offset, which saves the per-lane adds, made the kernel ~3% slower)
    // A rows of super step ss into A slot `slot`
    auto issue_a = [&](int ss, int slot) {
#pragma unroll
      for (int d = 0; d < S::DPW; ++d) {
        uint8_t* dst = als + slot * S::ASLOT + S::RPI * (S::DPW * wave + d) * S::AROWB;
        if constexpr (KT) {
          // chunks past K (a K tail) read the row's first chunk; their scales are zeroed
          const int ko = ss * SPAN + achk[d];
          dma16s(arsrc, 2u * (arow[d] + (uint32_t)(ko < K ? ko : 0)), dst);
        } else {
          dma16s(arsrc, 2u * (arow[d] + (uint32_t)(ss * SPAN + achk[d])), dst);
        }
      }
    };
    auto issue = [&](int ss, u32x4* o, int t) {
      if constexpr (!AR) {
        issue_a(ss, (ss - ss0) % S::NSLOT);
        if (t >= 0)
          issue_s(t / S::SBLK + 2, t % S::SBLK);
        else
          issue_s(1, t + S::SBLK);
      }
      if constexpr (KT) {
        const int kl = ss * SPAN + S::G * q;
        const uint32_t kc = kl < K ? (uint32_t)kl / 2 : 0u;
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) o[cg] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, coff[cg] + kc, 0, 0);
      } else {
        const uint32_t kc = (uint32_t)(ss * SPAN + S::G * q) / 2;
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) o[cg] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, coff[cg] + kc, 0, 0);
      }
    };
    f32x4 acc[NRG][CG];
#pragma unroll
    for (int r = 0; r < NRG; ++r)
#pragma unroll
      for (int i = 0; i < CG; ++i) acc[r][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one super step: wait for its loads (only those of the next NSET - 2
    // steps may still be in flight; the barrier publishes the other
    // wavefronts' A and frees the A slot of step ss - 1, which step
    // ss + NSET - 1 may reuse), issue step ss + NSET - 1, then per 16-value
    // block: read the A fragments and scales, convert the codes, MFMA chains
    // and scale FMAs
    auto step = [&](int ss, const u32x4* cur, u32x4* next) {
      if constexpr (AR) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSET - 2) * CG) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSET - 2) * (S::NWL + S::DPW)) : "memory");
        __builtin_amdgcn_s_barrier();
      }
      issue(clampss(ss + NSET - 1), next, ss - ss0);
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t slot = lds_base + (AR ? ss - ss0 : (ss - ss0) % S::NSLOT) * S::ASLOT;
      const uint32_t sslot = sbase + (AR ? 0 : (((ss - ss0) / S::SBLK) % 3) * S::SSLOT) + ((ss - ss0) % S::SBLK) * 16;
      const bool kin = !KT || ss * SPAN + S::G * q < K;  // false only in a K tail
      // block scales 2q, 2q + 1 of this lane's columns (bytes 0, 1 of a u16)
      uint32_t scr[CG];
      {
        const uint32_t sa = sslot + scoff;
        scr[0] = lds_read_u16o<0>(sa);
        scr[1] = lds_read_u16o<1024>(sa);
        scr[2] = lds_read_u16o<2048>(sa);
        scr[3] = lds_read_u16o<3072>(sa);
        static_assert(CG == 4, "four column groups");
      }
      float sf[CG][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        u32x4 af[NRG][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t aa = slot + aoff[2 * sb + h];
          af[0][h] = lds_read16o<0>(aa);
          if constexpr (NRG > 1) af[1][h] = lds_read16o<4 * S::AROWB>(aa);
        }
        if constexpr (NRG == 1)
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(af[0][0]), "+v"(af[0][1]), "+v"(scr[0]), "+v"(scr[1]), "+v"(scr[2]), "+v"(scr[3])
                       :
                       : "memory");
        else
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(af[0][0]), "+v"(af[0][1]), "+v"(af[1][0]), "+v"(af[1][1]), "+v"(scr[0]), "+v"(scr[1]),
                         "+v"(scr[2]), "+v"(scr[3])
                       :
                       : "memory");
        if (sb == 0) {  // as fp32 (exact), zero past K
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) {
            const f32x2 sp = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(scr[cg], 1.0f, false);
            sf[cg][0] = kin ? sp.x : 0.f;
            sf[cg][1] = kin ? sp.y : 0.f;
          }
        }
        // MFMA chains (4 K values each, 4 per 16-value block) of CI column
        // groups x NRG row groups side by side: a lone chain waits out the
        // full MFMA latency at every link
#pragma unroll
        for (int cb = 0; cb < CG / CI; ++cb) {
          f32x4 t[CI][NRG];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int ci = 0; ci < CI; ++ci) {
              const uint32_t d = cur[cb * CI + ci][2 * sb + (m >> 1)];
              const u32x2 bv = (m & 1) ? e2m1_bf16_4<2>(d) : e2m1_bf16_4<0>(d);
#pragma unroll
              for (int r = 0; r < NRG; ++r) {
                const f32x4 c = m == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : t[ci][r];
                t[ci][r] = (m & 1) ? mfma4h<1>(af[r][m >> 1], bv, c) : mfma4h<0>(af[r][m >> 1], bv, c);
              }
            }
          }
#pragma unroll
          for (int ci = 0; ci < CI; ++ci)
#pragma unroll
            for (int r = 0; r < NRG; ++r) acc[r][cb * CI + ci] += sf[cb * CI + ci][sb] * t[ci][r];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // the previous pass's LDS reads and direct loads are done before the
    // slots are refilled; then the first scale blocks and NSET - 1 steps
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (AR) {
      // the scale block and the A rows of every step, before the first codes
#pragma unroll 1
      for (int st = 0; st < S::SBLK; ++st) issue_s(0, st);
#pragma unroll 1
      for (int s = ss0; s < ss1; ++s) issue_a(s, s - ss0);
    } else {
      // (only the blocks this K range reads: at most one for 8 super steps)
      const int nblk = (ss1 - ss0 + S::SBLK - 1) / S::SBLK;
#pragma unroll 1
      for (int st = 0; st < 2 * S::SBLK; ++st)
        if (st / S::SBLK < nblk) issue_s(st / S::SBLK, st % S::SBLK);
    }
    // AR: once the first steps' codes are issued, the direct loads before them
    // have landed when only those codes are outstanding; the barrier publishes
    // every wavefront's A rows
    auto publish = [&]() {
      if constexpr (AR) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSET - 1) * CG) : "memory");
        __syncthreads();
      }
    };
    int ss = ss0;
    if constexpr (NSET == 4) {
      u32x4 w0[CG], w1[CG], w2[CG], w3[CG];
      issue(ss0, w0, -3);
      issue(clampss(ss0 + 1), w1, -2);
      issue(clampss(ss0 + 2), w2, -1);
      publish();
      for (; ss + 3 < ss1; ss += 4) {
        step(ss, w0, w3);
        step(ss + 1, w1, w0);
        step(ss + 2, w2, w1);
        step(ss + 3, w3, w2);
      }
      // w0, w1, w2 hold steps ss, ss + 1, ss + 2
      if (ss < ss1) step(ss, w0, w3);
      if (ss + 1 < ss1) step(ss + 1, w1, w0);
      if (ss + 2 < ss1) step(ss + 2, w2, w1);
    } else if constexpr (NSET == 2) {
      u32x4 w0[CG], w1[CG];
      issue(ss0, w0, -1);
      publish();
      for (; ss + 1 < ss1; ss += 2) {
        step(ss, w0, w1);
        step(ss + 1, w1, w0);
      }
      if (ss < ss1) step(ss, w0, w1);  // w0 holds step ss
    } else {
      u32x4 w0[CG], w1[CG], w2[CG];
      issue(ss0, w0, -2);
      issue(clampss(ss0 + 1), w1, -1);
      publish();
      for (; ss + 2 < ss1; ss += 3) {
        step(ss, w0, w2);
        step(ss + 1, w1, w0);
        step(ss + 2, w2, w1);
      }
      if (ss < ss1) step(ss, w0, w2);  // w0 holds step ss, w1 step ss + 1
      if (ss + 1 < ss1) step(ss + 1, w1, w0);
    }

    // epilogue: add the eight K ranges' partial sums; then lane (q, c8) holds
    // rows 4 rg + 0..3 of column colv[cg], and lanes q < 4 store row 4 rg + q
    const float gsc = a.w_gscale[e];
    float* pbase = a.ksplit > 1 ? a.part + (size_t)split * a.part_stride : nullptr;
#pragma unroll
    for (int r = 0; r < NRG; ++r) {
      float v[CG];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        f32x4 t = acc[r][cg];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          t[i] += __shfl_xor(t[i], 8);
          t[i] += __shfl_xor(t[i], 16);
          t[i] += __shfl_xor(t[i], 32);
        }
        v[cg] = ((q & 3) == 0 ? t[0] : (q & 3) == 1 ? t[1] : (q & 3) == 2 ? t[2] : t[3]) * gsc;
      }
      const int m = mc + 4 * r + q;
      if (q >= 4 || m >= cnt || !tile_ok) continue;
      if (pbase) {  // split K: scaled fp32 partial sums
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) {
          const int col = column(cg, c8);
          if (col < N) pbase[(size_t)(r0 + m) * N + col] = v[cg];
        }
      } else if (GATE_UP) {
#pragma unroll
        for (int cg = 0; cg < CG / 2; ++cg)
          a.h_out[(size_t)(r0 + m) * a.I + column(cg, c8)] =
              (uint16_t)f32_to_bf16_bits(silu(v[cg]) * v[cg + CG / 2]);
      } else {
#pragma unroll
        for (int cg = 0; cg < CG; ++cg) {
          const int col = column(cg, c8);
          if (col < N) store_rows(a.y_out + (size_t)(r0 + m) * N + col, v[cg]);
        }
      }
    }
  };

  for (int mc = 0; mc < cnt; mc += S::AROWS) {
    const int nrg = (cnt - mc + 3) / 4;  // row groups holding rows
    if (nrg <= 1)
      pass(mc, std::integral_constant<int, 1>{});
    else
      pass(mc, std::integral_constant<int, 2>{});
  }
}

// NVFP4: 8 rows per pass at any row count (measured at 12 and 16 rows per
// expert: two 8-row passes beat one 16-row pass by 20%, whose kernel wants
// ~400 registers and spills at two workgroups per CU, and by 7% with one
// workgroup per CU and no spills)
template <bool GU, bool KT, bool AR>
void launch_fp4_k(dim3 grid, const StreamGemmArgs& a, hipStream_t st) {
  stream_fp4_kernel<2, GU, KT, AR><<<grid, 256, 0, st>>>(a);
}
template <bool GU>
void launch_fp4(dim3 grid, const StreamGemmArgs& a, hipStream_t st) {
  // K range of a workgroup, in super steps
  const int nss = (a.K + Fp4Shape<2>::SPAN - 1) / Fp4Shape<2>::SPAN;
  const bool ar = (a.ksplit > 1 ? a.ksteps : nss) <= Fp4Shape<2>::SBLK;
  if (a.K % Fp4Shape<2>::SPAN != 0) {
    if (ar)
      launch_fp4_k<GU, true, true>(grid, a, st);
    else
      launch_fp4_k<GU, true, false>(grid, a, st);
  } else {
    if (ar)
      launch_fp4_k<GU, false, true>(grid, a, st);
    else
      launch_fp4_k<GU, false, false>(grid, a, st);
  }
}

}  // namespace

int stream_q_cols(int wfmt) { return wfmt == W_FP8 ? KmShape<W_FP8>::COLS : Fp4Shape<2>::COLS; }

int stream_q_k_step(int wfmt) { return wfmt == W_FP8 ? KmShape<W_FP8>::SPAN : Fp4Shape<2>::SPAN; }

hipError_t launch_stream_q(int wfmt, bool gate_up, dim3 grid, const StreamGemmArgs& a, hipStream_t st) {
  switch (wfmt) {
    case W_FP8:
      if (gate_up)
        stream_kmajor_kernel<W_FP8, true><<<grid, 256, 0, st>>>(a);
      else
        stream_kmajor_kernel<W_FP8, false><<<grid, 256, 0, st>>>(a);
      break;
    case W_FP4:
      if (gate_up)
        launch_fp4<true>(grid, a, st);
      else
        launch_fp4<false>(grid, a, st);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
