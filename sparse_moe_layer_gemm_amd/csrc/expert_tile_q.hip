// Grouped SwiGLU expert GEMMs with FP8 (E4M3) and NVFP4 weights for many
// rows per expert, on gfx950 MFMA, in both quantised modes: weights
// dequantised exactly to bf16 (bf16 MFMA; the pages' NVFP4 variant with BF16
// activations, vLLM recipe "reflection/Beam-1.0-501B-A23B", Guide >
// Variants), and the fp8-MFMA mode (activations quantised to E4M3 in-kernel).
// The tile pipeline is that of the bf16 tiled kernels (expert_tile.hip).
#include "tile_common.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ FP8 / NVFP4 weights
// Same tiling for K-contiguous quantised weights ([E, N, K] E4M3 codes, or
// [E, N, K/2] E2M1 codes with one E4M3 scale per 16 K values): per K step a
// column's codes (16 B for E2M1, 32 B for E4M3) and, for E2M1, the dword of
// block scales holding this step's two come in by direct loads next to the A
// tile. B fragments are read as one contiguous run per lane and converted to
// bf16 in registers: E4M3 -> bf16 is exact in the hardware converter; E2M1
// codes become fp32 in the converter and one fp32 multiply applies the E4M3
// block scale (the product has at most 6 significant bits, so it is exact, as
// is its bf16 upper half). Per-channel
// (E4M3) and per-expert (E2M1) fp32 scales multiply the accumulators in the
// epilogue. Within a K step, lane half kh takes K 16*kh .. 16*kh+15 (MFMA s
// the 8 from 16*kh + 8*s), so a lane's codes are contiguous and, for E2M1,
// each lane needs a single block scale per step.
// The 128 x 512 tile runs 8 wavefronts side by side along N, each 128 rows x
// 64 columns (128 accumulators), two per SIMD: every weight column is
// converted by exactly one wavefront, and while one wavefront of a SIMD
// converts its codes (VALU) the other can issue its MFMAs.
template <int WF>
struct QShape {
  using T = TileShape<1, 8>;
  static constexpr int NW = 8;
  static constexpr int BM = T::BM, BN = T::BN, WN = T::WN, JT = T::JT;
  static constexpr int COL = WF == W_FP4 ? 16 : 32;   // code bytes per column per K step
  static constexpr int A_STAGE = 160 * TBK * 2;       // up to 160 rows x 64 B (a merged tail)
  // codes arrive as 64 B per column (CSS K steps) in code stages of the whole
  // tile's columns, three in LDS; a load instruction covers 16 columns x 64 B
  static constexpr int CSS = 64 / COL;                // K steps per code stage
  static constexpr int CSLOT = BN * 64;               // bytes of a code stage
  static constexpr int NCS = 3;
  // NVFP4 block scales: 16 B per column (8 K steps) per scale stage, three in LDS
  static constexpr int SSS = 8;                       // K steps per scale stage
  static constexpr int SSLOT = WF == W_FP4 ? BN * 16 : 0;
  static constexpr int NSS = 3;
  static constexpr int C_OFF = NSTAGE * A_STAGE;      // code stages after the A stages
  static constexpr int S_OFF = C_OFF + NCS * CSLOT;   // then the scale stages
  static constexpr int PIPE = S_OFF + NSS * SSLOT;
  static constexpr int EPI = NW * 8192;               // epilogue strips (32 x 64 fp32 each)
  static constexpr int LDS = PIPE > EPI ? PIPE : EPI;
  static constexpr int QA = A_STAGE / 1024 / NW;      // 1 KB A loads per wavefront
  static constexpr int QB = CSLOT / CSS / 1024 / NW;  // code loads per wavefront per K step
  // loads per wavefront per K step, not counting the scale load one K step in 8 adds
  static constexpr int PER_STEP = QA + QB;
  static_assert(QA == 1 && NW * QB * CSS * 16 == BN, "every column's code stage loaded once");
  static_assert(PIPE <= 160 * 1024, "LDS");
};

// 16-byte LDS read at addr + OFF (an immediate offset), valid after an
// explicit lgkmcnt wait that takes the result as an operand
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128o(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_b64o(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ uint32_t lds_b32o(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
// the NF A fragments of one K half: rows 32 i + l32 sit 2 KB apart at the
// same swizzled chunk (the swizzle depends on row bits 2-3 only)
template <int NF>
__device__ __forceinline__ void lds_a_frags(u32x4 (&a)[NF], uint32_t addr) {
  static_assert(NF == 4 || NF == 5, "four or five row fragments");
  a[0] = lds_b128o<0>(addr);
  a[1] = lds_b128o<2048>(addr);
  a[2] = lds_b128o<4096>(addr);
  a[3] = lds_b128o<6144>(addr);
  if constexpr (NF == 5) a[4] = lds_b128o<8192>(addr);
}

// raw codes of one column per lane per K step: 8 B (E2M1) or 16 B (E4M3)
template <int WF> struct QRaw { typedef u32x4 type; };
template <> struct QRaw<W_FP4> { typedef u32x2 type; };
// One 128-row (NF = 4) or up to 160-row (NF = 5: an expert's last tile
// with its <= 32-row tail merged in) x 512-column tile of a quantised
// grouped GEMM.
template <int WF, bool GATE_UP, int NF>
__device__ __forceinline__ void tile_q_body(const StreamGemmArgs& a, uint8_t* smem, int e, int m0,
                                            int nt, int r0, int cnt) {
  using S = QShape<WF>;
  constexpr int JT = S::JT;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wn = wave;
  const int K = a.K, N = a.N;

  // A: as in the bf16 kernel (gathered rows, 16 rows per 1 KB load; wavefront
  // w loads rows 16 w .. 16 w + 15, and with a fifth row fragment wavefronts
  // 0 and 1 also rows 128 + 16 w ..)
  constexpr int NX = NF > 4 ? 1 : 0;  // extra A loads of wavefronts 0 and 1
  const uint16_t* asrc[1 + NX];
#pragma unroll
  for (int q = 0; q <= NX; ++q) {
    const int row = 128 * q + 16 * (q ? (wave & 1) : wave) + (lane >> 2);
    const int lg = (lane & 3) ^ ((row >> 2) & 3);
    size_t grow = 0;
    if (m0 + row < cnt)
      grow = GATE_UP ? (size_t)(a.sorted_pair[r0 + m0 + row] / a.k) : (size_t)(r0 + m0 + row);
    asrc[q] = a.a + grow * K + 8 * lg;
  }
  // matrix column of LDS column c (gate/up: BN/2 gate, then the matching up)
  auto mcol = [&](int c) -> int {
    if (GATE_UP) {
      const int gc = nt * (S::BN / 2) + (c < S::BN / 2 ? c : c - S::BN / 2);
      if (gc >= a.I) return 0;  // clamped: feeds accumulators never stored
      return c < S::BN / 2 ? gc : a.I + gc;
    }
    const int col = nt * S::BN + c;
    return col < N ? col : 0;
  };
  const uint8_t* wq = static_cast<const uint8_t*>(a.w);
  const int row_bytes = WF == W_FP4 ? K / 2 : K;
  // code stage cs holds K steps CSS cs .. CSS cs + CSS - 1 of every column:
  // 16-column block ib at ib * 1024, 16 B chunk q of the stage's 64 B at
  // + 256 q, column c of the block at + 16 c (a load's lane l is chunk l / 16
  // of column l % 16). Wavefront w loads blocks 4 w .. 4 w + 3, QB per K step.
  // A wavefront's blocks are consecutive matrix columns of one side (gate,
  // up, or the down GEMM's N): block p's column is col0 + 16 p, columns past
  // the side's end read its last column (they feed accumulators never
  // stored), so a block's address is arithmetic in p rather than a runtime
  // index into per-block pointers.
  // the expert's codes as a buffer (its byte size fits 31 bits, checked by the host)
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wq + (size_t)e * N * row_bytes), (short)0, N * row_bytes, 0x00020000);
  int col0, colmax;
  {
    const int c = 64 * wave + (lane & 15);  // LDS column of block 0
    if (GATE_UP) {
      const bool up = c >= S::BN / 2;
      col0 = (up ? a.I : 0) + nt * (S::BN / 2) + (up ? c - S::BN / 2 : c);
      colmax = (up ? 2 * a.I : a.I) - 1;
    } else {
      col0 = nt * S::BN + c;
      colmax = N - 1;
    }
  }
  const uint32_t kq = 16 * (lane >> 4);
  auto code_off = [&](int p) -> uint32_t {
    const int col = col0 + 16 * p;
    return (uint32_t)(col < colmax ? col : colmax) * (uint32_t)row_bytes + kq;
  };
  // scale stage t holds 16 B per column (K steps 8 t .. 8 t + 7) at 16 column;
  // wavefront w loads its 64 columns' 16 B, lane l column 64 w + l
  const uint8_t* ssrc = WF == W_FP4 ? static_cast<const uint8_t*>(a.w_scale) +
                                          ((size_t)e * N + mcol(64 * wave + lane)) * (size_t)(K / 16)
                                    : nullptr;
  // code piece p of stage cs (chunks past the row, in a K tail, read its start)
  // (chunks past the row, in a K tail, read the next row's bytes or, past
  // the buffer, zeros: they belong to K steps that are never computed)
  auto load_code = [&](int cs, int p) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc,
                                             (__attribute__((address_space(3))) void*)(smem + S::C_OFF +
                                                 (cs % S::NCS) * S::CSLOT + (4 * wave + p) * 1024),
                                             16, code_off(p), 64 * cs, 0, 0);
  };
  auto load_scale = [&](int t) {
    const int ko = 16 * t;
    dma16(ssrc + (ko + 16 <= K / 16 ? ko : 0), smem + S::S_OFF + (t % S::NSS) * S::SSLOT + 64 * wave * 16);
  };
  // the loads issued for K step kt (three steps ahead): one scale stage piece
  // (NVFP4, wavefront kt % 8, for the next scale stage), the A rows, and
  // piece kt % CSS of the next code stage
  auto issue = [&](int kt, int st) {
    if (WF == W_FP4 && (kt & 7) == wave) load_scale(kt / S::SSS + 1);
    if (NX && wave < 2) dma16(asrc[NX] + kt * TBK, smem + st * S::A_STAGE + (128 + 16 * wave) * 64);
    dma16(asrc[0] + kt * TBK, smem + st * S::A_STAGE + 16 * wave * 64);
#pragma unroll
    for (int q = 0; q < S::QB; ++q) load_code(kt / S::CSS + 1, (kt % S::CSS) * S::QB + q);
  };

  f32x16 acc[NF][JT];
#pragma unroll
  for (int i = 0; i < NF; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS column of this wave's 32-column tile j (gate/up: its gate tile, then
  // the matching up tile)
  auto bcol = [&](int j) -> int {
    if (GATE_UP) return j == 0 ? 32 * wn : S::BN / 2 + 32 * wn;
    return 64 * wn + 32 * j;
  };
  const int l32 = lane & 31, kh = lane >> 5;
  const uint32_t lds0 = (uint32_t)(size_t)(lds_u8*)smem;
  uint32_t aoff[2], boff[JT], soff[JT];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) aoff[s2] = a_off(l32, 2 * kh + s2);  // row fragment 0
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int c = bcol(j) + l32;
    // this lane's 8 B (E2M1) or 16 B (E4M3) of column c at K step 0 of a code stage
    boff[j] = (c >> 4) * 1024 + 16 * (c & 15) + (WF == W_FP4 ? 8 * kh : 256 * kh);
    soff[j] = c * 16 + kh;
  }
  // first half of a K step: A (K half 0), the codes and the block scales;
  // second half: A (K half 1)
  struct FragQ0 {
    u32x4 a[NF];
    typename QRaw<WF>::type b[JT];
    uint32_t sc[JT];
  };
  struct FragQ1 {
    u32x4 a[NF];
  };
  auto read0 = [&](FragQ0& f, int st, int kt) {
    const uint32_t cbase = lds0 + S::C_OFF + ((kt / S::CSS) % S::NCS) * S::CSLOT + (kt % S::CSS) * (S::COL / 16) * 256;
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      if constexpr (WF == W_FP4)
        f.b[j] = lds_b64(cbase + boff[j]);
      else
        f.b[j] = lds_b128(cbase + boff[j]);
    }
    if (WF == W_FP4) {
      // block 2 kt + kh: byte 2 (kt % 8) + kh of the column's 16 B
      const uint32_t sbase = lds0 + S::S_OFF + ((kt / S::SSS) % S::NSS) * S::SSLOT + 2 * (kt % S::SSS);
#pragma unroll
      for (int j = 0; j < JT; ++j) f.sc[j] = lds_byte(sbase + soff[j]);
    }
    lds_a_frags<NF>(f.a, lds0 + st * S::A_STAGE + aoff[0]);
  };
  auto read1 = [&](FragQ1& f, int st) { lds_a_frags<NF>(f.a, lds0 + st * S::A_STAGE + aoff[1]); };
  // (the fifth A fragment, when there is one, as an operand of its own wait)
#define MOE_LGK_WAIT0(f, pending)                                                              \
  do {                                                                                         \
    if constexpr (NF == 5)                                                                     \
      asm volatile("s_waitcnt lgkmcnt(%9)"                                                    \
                   : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]),     \
                     "+v"(f.b[1]), "+v"(f.sc[0]), "+v"(f.sc[1]), "+v"(f.a[NF - 1])            \
                   : "n"(pending)                                                              \
                   : "memory");                                                                \
    else                                                                                       \
      asm volatile("s_waitcnt lgkmcnt(%8)"                                                    \
                   : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]),     \
                     "+v"(f.b[1]), "+v"(f.sc[0]), "+v"(f.sc[1])                                \
                   : "n"(pending)                                                              \
                   : "memory");                                                                \
  } while (0)
  // the second-half wait also covers the next step's codes and block scales
  // (issued before its A reads), which the second half converts
#define MOE_LGK_WAIT1B(f, g, pending)                                                          \
  do {                                                                                         \
    if constexpr (NF == 5)                                                                     \
      asm volatile("s_waitcnt lgkmcnt(%9)"                                                    \
                   : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.a[NF - 1]), \
                     "+v"(g.b[0]), "+v"(g.b[1]), "+v"(g.sc[0]), "+v"(g.sc[1])                  \
                   : "n"(pending)                                                              \
                   : "memory");                                                                \
    else                                                                                       \
      asm volatile("s_waitcnt lgkmcnt(%8)"                                                    \
                   : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(g.b[0]),     \
                     "+v"(g.b[1]), "+v"(g.sc[0]), "+v"(g.sc[1])                                \
                   : "n"(pending)                                                              \
                   : "memory");                                                                \
  } while (0)
  // codes of K half s2 -> bf16 fragments bq[s2]; an NVFP4 lane's block
  // scales (one per column tile and K step) as fp32, both in one conversion.
  // Each code's E2M1 value times its E4M3 scale has at most 6 significant
  // bits, so the fp32 product, and its bf16 upper half, are exact.
  u32x4 bq[2][JT];
  float sfv[JT];
  auto scales_f32 = [&](const FragQ0& f) {
    if constexpr (WF == W_FP4) {
      static_assert(JT == 2, "two column tiles: both block scales in one conversion");
      const f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(f.sc[0] | (f.sc[1] << 8), 1.0f, false);
      sfv[0] = sv.x;
      sfv[1] = sv.y;
    }
  };
  auto dequant_half = [&](const FragQ0& f, int s2) {
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      if constexpr (WF == W_FP4)
        bq[s2][j] = fp4_frag(f.b[j][s2], 1.0f, sfv[j]);
      else
        bq[s2][j] = fp8_frag(f.b[j][2 * s2], f.b[j][2 * s2 + 1]);
    }
  };
  auto mfma_half = [&](const u32x4 (&af)[NF], int s2) {
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int i = 0; i < NF; ++i) acc[i][j] = mfma32(af[i], bq[s2][j], acc[i][j]);
  };
  // one MFMA, then a few conversion instructions, in turn: the conversion of
  // the other K half runs in the shadow of this half's MFMAs
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < NF * JT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
    }
  };
  // Pipeline as in the bf16 kernel: "step kt+1 landed" is vmcnt(PER_STEP)
  // once three steps are in flight (a K step's scale load is issued first, so
  // counting it out only waits for it early); f1 (4 reads) is read while f0's
  // MFMAs run, f0 of the next step (6 or 8 reads) while f1's run. The B
  // fragments of a K half are converted while the MFMAs of the other half
  // run: half 1 of step kt during the first half's MFMAs, half 0 of step
  // kt + 1 (its codes read mid-step) during the second half's. The first
  // code and scale stages are loaded before the first three steps.
  const int nk = K / TBK;
  if (WF == W_FP4) load_scale(0);
#pragma unroll
  for (int p = 0; p < S::CSS * S::QB; ++p) load_code(0, p);
  issue(0, 0);
  issue(nk > 1 ? 1 : nk - 1, 1);
  issue(nk > 2 ? 2 : nk - 1, 2);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * S::PER_STEP) : "memory");
  __builtin_amdgcn_s_barrier();
  FragQ0 f0;
  FragQ1 f1;
#pragma unroll
  for (int j = 0; j < JT; ++j) f0.sc[j] = 0u;
  read0(f0, 0, 0);
  MOE_LGK_WAIT0(f0, NF);  // codes and scales of step 0 (its A may still be in flight)
  scales_f32(f0);
  dequant_half(f0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    read1(f1, kt % NSTAGE);
    MOE_LGK_WAIT0(f0, NF);
    mfma_half(f0.a, 0);
    dequant_half(f0, 1);
    interleave();
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(S::PER_STEP) : "memory");
    __builtin_amdgcn_s_barrier();
    read0(f0, (kt + 1) % NSTAGE, kt + 1);
    MOE_LGK_WAIT1B(f1, f0, NF);
    scales_f32(f0);
    mfma_half(f1.a, 1);
    dequant_half(f0, 0);
    interleave();
    // (a use here keeps the conversion in this block, beside the MFMAs,
    // rather than sunk past the branch below to its first real use)
#pragma unroll
    for (int j = 0; j < JT; ++j) asm volatile("" ::"v"(bq[0][j]));
    // the stage of step kt - 1 is free since the barrier; issued last, so
    // that the scale load's branch ends the loop body
    issue(kt + 3 < nk ? kt + 3 : nk - 1, (kt + 3) % NSTAGE);
  }
  MOE_LGK_WAIT0(f0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef MOE_LGK_WAIT0
#undef MOE_LGK_WAIT1B
  __builtin_amdgcn_s_barrier();

  // ---- epilogue through LDS (each wavefront its own strip), scales applied first
  const float gsc = WF == W_FP4 ? a.w_gscale[e] : 1.f;
  const float* chs = WF == W_FP8 ? static_cast<const float*>(a.w_scale) + (size_t)e * N : nullptr;
  auto tile_row = [&](int r) { return 8 * (r >> 2) + 4 * kh + (r & 3); };
  if (GATE_UP) {
    const float sg = WF == W_FP8 ? chs[mcol(bcol(0) + l32)] : gsc;
    const float su = WF == W_FP8 ? chs[mcol(bcol(1) + l32)] : gsc;
    uint16_t* strip = reinterpret_cast<uint16_t*>(smem + wave * 4096);  // 32 x 32 bf16
#pragma unroll
    for (int i = 0; i < NF; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        strip[tile_row(r) * 32 + l32] =
            (uint16_t)f32_to_bf16_bits(silu(acc[i][0][r] * sg) * (acc[i][1][r] * su));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < 2; ++t) {  // 32 rows x 4 chunks of 16 B
        const int c = lane + 64 * t, rr = c >> 2, ch = c & 3;
        const int m = m0 + 32 * i + rr;
        const int col = nt * (S::BN / 2) + 32 * wn + 8 * ch;
        const u32x4 v = *reinterpret_cast<const u32x4*>(strip + rr * 32 + 8 * ch);
        if (m < cnt && col < a.I)
          *reinterpret_cast<u32x4*>(a.h_out + (size_t)(r0 + m) * a.I + col) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else {
    float sd[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) sd[j] = WF == W_FP8 ? chs[mcol(bcol(j) + l32)] : gsc;
    float* strip = reinterpret_cast<float*>(smem + wave * 8192);  // 32 x 64 fp32
    const bool compact = a.y16 != nullptr;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
#pragma unroll
      for (int j = 0; j < JT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) strip[tile_row(r) * 64 + 32 * j + l32] = acc[i][j][r] * sd[j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (compact) {  // compact rows: one 64-column scale block per strip row
        store_rows16<64>(strip, lane, m0 + 32 * i, cnt, nt * S::BN + 64 * wn, N, (size_t)r0,
                         a.y16, a.y16_scale);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {  // 32 rows x 16 chunks of 16 B
          const int c = lane + 64 * t, rr = c >> 4, ch = c & 15;
          const int m = m0 + 32 * i + rr;
          const int col = nt * S::BN + 64 * wn + 4 * ch;
          const f32x4 v = *reinterpret_cast<const f32x4*>(strip + rr * 64 + 4 * ch);
          if (m < cnt && col < N) store_rows(a.y_out + (size_t)(r0 + m) * N + col, v);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

template <int WF, bool GATE_UP>
__global__ __launch_bounds__(512, 1) void tile_q_kernel(StreamGemmArgs a,
                                                        const int32_t* __restrict__ tile_e,
                                                        const int32_t* __restrict__ tile_m0,
                                                        const int32_t* __restrict__ n_tiles_p,
                                                        int NT) {
  using S = QShape<WF>;
  __shared__ __align__(1024) uint8_t smem[S::LDS];

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
  // an expert's last tile holds up to 160 rows (tile_table_kernel merges a
  // tail of <= 32 rows into it)
  if (cnt - m0 > 128)
    tile_q_body<WF, GATE_UP, 5>(a, smem, e, m0, nt, r0, cnt);
  else
    tile_q_body<WF, GATE_UP, 4>(a, smem, e, m0, nt, r0, cnt);
}

// ------------------------------------------------------------------ fp8-MFMA mode
// Both expert GEMMs on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32
// accumulate, 64 K per instruction at twice the bf16 rate). Operands:
//  - gate/up A: x as E4M3 codes with one fp32 scale per token (applied with
//    the weight scales in the epilogue, before SwiGLU);
//  - down A: h as E4M3 codes with one power-of-two (E8M0) scale per row and
//    128-column block, handed to the MFMA, which applies it exactly;
//  - B: FP8 weights as stored, or NVFP4 weights re-encoded per 32-deep K
//    block as RNE_e4m3(e2m1 * s_blk * 2^-s) in registers, s = (the exponent
//    field of the block's larger E4M3 scale) - 12 (the converter gives e2m1
//    times the scale's power of two times 2^-s, an fp32 multiply its mantissa
//    factor, and the hardware f32 -> E4M3 conversion rounds to nearest even);
//    2^s is the lane's E8M0 B scale in the MFMA, so the re-encoding is as
//    precise for any range of block scales.
// Lane half g takes K 32g .. 32g+31 of each 64-deep step for both operands;
// the scale of a down-GEMM row is the same over the whole step, so the K
// order inside the step is free.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

template <int WF, int WM>
struct F8Shape {
  using T = TileShape<WM>;
  static constexpr int BM = T::BM, BN = T::BN, WN = T::WN;
  static constexpr int A_STAGE = BM * 64;                            // 64 codes per row
  // E4M3 codes: 64 B per column per K step, in the pipeline stages. E2M1
  // codes: 64 B per column per two K steps (code stages of the whole tile's
  // columns, three in LDS, a load covering 16 columns), and their block
  // scales 16 B per column per four K steps (scale stages, three in LDS, a
  // load covering 64 columns).
  static constexpr int B_STAGE = WF == W_FP8 ? BN * 64 : 0;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int CSLOT = WF == W_FP4 ? BN * 64 : 0;
  static constexpr int SSLOT = WF == W_FP4 ? BN * 16 : 0;
  static constexpr int ROWB = 32;                                    // bytes of row data per row
  static constexpr int ROWDATA = BM * ROWB;
  static constexpr int SIDE = 3 * CSLOT + 3 * SSLOT;                 // E2M1 code and scale stages
  static constexpr int NST = (4 * STAGE + SIDE + ROWDATA <= 163840) ? 4 : 3;
  static constexpr int C_OFF = NST * STAGE;
  static constexpr int S_OFF = C_OFF + 3 * CSLOT;
  static constexpr int PIPE = NST * STAGE + SIDE > 65536 ? NST * STAGE + SIDE : 65536;
  static constexpr int LDS = PIPE + ROWDATA;
  static constexpr int QA = BM / 64;                                 // 1 KB A loads per wavefront
  static constexpr int QB = WF == W_FP8 ? BN / 64 : BN / 128;        // 1 KB code loads per wavefront
  // loads per wavefront per K step (E2M1: not counting the scale load every
  // other K step, issued first, so that counting it out only waits for it early)
  static constexpr int PER_STEP = QA + QB;
  static_assert(WF == W_FP8 || 4 * QB * 2 * 16 == BN, "E2M1: every column's code stage loaded once");
  static_assert(WF == W_FP8 || BN == 512 || BN == 256, "E2M1: 8 or 4 scale loads per scale stage");
};

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 8 E2M1 codes (one dword) x block scale (p2 * fm8: the scale's power of two,
// times the block's shift, and its mantissa factor) -> 8 E4M3 codes (two dwords)
__device__ __forceinline__ void fp4_to_fp8(uint32_t d, float p2, float fm8, int32_t& o0,
                                           int32_t& o1) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, p2, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, p2, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, p2, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, p2, 3);
  // each first conversion writes the low half of a dword whose high half the
  // second writes: its "old" operand is one of its own (dead) inputs, whose
  // register the result can take, rather than a zero that needs a move
  const float p0 = v0.x * fm8, p1 = v0.y * fm8, p4 = v2.x * fm8, p5 = v2.y * fm8;
  int32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
  o0 = __builtin_amdgcn_cvt_pk_fp8_f32(v1.x * fm8, v1.y * fm8, r, true);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(p4, p5, __float_as_int(p4), false);
  o1 = __builtin_amdgcn_cvt_pk_fp8_f32(v3.x * fm8, v3.y * fm8, r, true);
}

template <int WF> struct F8Raw { typedef i32x8 type; };      // E4M3: 32 codes
template <> struct F8Raw<W_FP4> { typedef u32x4 type; };     // E2M1: 32 codes

template <int WF, bool GATE_UP, int WM>
__global__ __launch_bounds__(256, 1) void tile_f8_kernel(F8Args f8, StreamGemmArgs a,
                                                         const int32_t* __restrict__ tile_e,
                                                         const int32_t* __restrict__ tile_m0,
                                                         const int32_t* __restrict__ n_tiles_p,
                                                         int NT) {
  using S = F8Shape<WF, WM>;
  __shared__ __align__(1024) uint8_t smem[S::LDS];
  uint8_t* rowdata = smem + S::PIPE;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / S::WN, wn = wave % S::WN;

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
  const int nb = (K + 127) / 128;  // 128-column blocks of a down-GEMM row

  // per-row data: gate/up the token's fp32 activation scale; down the row's
  // E8M0 block scales, stored [block][slot] with slot = 4 * (32 wm + l32) + i
  // for tile row 128 wm + 32 i + l32, so a lane reads its four rows' scales of
  // a block as one dword (rows past the expert's end get neutral values)
  for (int r = tid; r < S::BM; r += 256) {
    const bool ok = m0 + r < cnt;
    if (GATE_UP) {
      const float sc = ok ? f8.x_scale[a.sorted_pair[r0 + m0 + r] / a.k] : 0.f;
      *reinterpret_cast<float*>(rowdata + r * S::ROWB) = sc;
    } else {
      const int slot = 4 * (32 * (r >> 7) + (r & 31)) + ((r >> 5) & 3);
      const uint8_t* src = f8.h_bscale + (size_t)(ok ? r0 + m0 + r : 0) * f8.h_bstride;
      for (int b = 0; b < nb; ++b) rowdata[b * S::BM + slot] = ok ? src[b] : (uint8_t)127;
    }
  }
  __syncthreads();

  // A: gathered code rows (64 B per row per step, as the bf16 A tile)
  const uint8_t* asrc[S::QA];
#pragma unroll
  for (int q = 0; q < S::QA; ++q) {
    const int row = (S::BM / 4) * wave + 16 * q + (lane >> 2);
    const int lg = (lane & 3) ^ ((row >> 2) & 3);
    size_t grow = 0;
    if (m0 + row < cnt)
      grow = GATE_UP ? (size_t)(a.sorted_pair[r0 + m0 + row] / a.k) : (size_t)(r0 + m0 + row);
    asrc[q] = f8.a8 + grow * K + 16 * lg;
  }
  auto mcol = [&](int c) -> int {
    if (GATE_UP) {
      const int gc = nt * (S::BN / 2) + (c < S::BN / 2 ? c : c - S::BN / 2);
      if (gc >= a.I) return 0;
      return c < S::BN / 2 ? gc : a.I + gc;
    }
    const int col = nt * S::BN + c;
    return col < N ? col : 0;
  };
  const uint8_t* wq = static_cast<const uint8_t*>(a.w);
  // B: E4M3 codes like A (16 columns x 64 B per load, swizzled granules);
  // E2M1 codes 32 B per column (two lanes per column), scale dwords one per column
  // E2M1: code stage cs holds K steps 2 cs, 2 cs + 1 of every column (64 B):
  // 16-column block ib at ib * 1024, 16 B chunk q at + 256 q, column c of the
  // block at + 16 c (a load's lane l is chunk l / 16 of column l % 16);
  // wavefront w loads blocks 2 QB w .. +2 QB, QB per K step. Scale stage t
  // holds 16 B per column (K steps 4 t .. 4 t + 3) at 16 column; its loads
  // cover 64 columns each.
  const uint8_t* bsrc[WF == W_FP8 ? S::QB : 2 * S::QB];
  if constexpr (WF == W_FP8) {
#pragma unroll
    for (int q = 0; q < S::QB; ++q) {
      const int col = (S::BN / 4) * wave + 16 * q + (lane >> 2);
      const int lg = (lane & 3) ^ ((col >> 2) & 3);
      bsrc[q] = wq + ((size_t)e * N + mcol(col)) * K + 16 * lg;
    }
  } else {
#pragma unroll
    for (int p = 0; p < 2 * S::QB; ++p)
      bsrc[p] = wq + ((size_t)e * N + mcol(16 * (2 * S::QB * wave + p) + (lane & 15))) * (size_t)(K / 2) +
                16 * (lane >> 4);
  }
  constexpr int NSP = WF == W_FP4 ? S::BN / 64 : 1;  // scale loads per scale stage
  const uint8_t* ssrc = WF == W_FP4 ? static_cast<const uint8_t*>(a.w_scale) + (size_t)e * N * (size_t)(K / 16)
                                    : nullptr;
  // E2M1 code piece p (of this wavefront's 2 QB) of code stage cs; chunks past
  // the row (a K tail) read the row's start
  // (hf: which half of the pieces, q: the piece within it; selected by value,
  // not by a runtime index into the pointer array, which costs indexed moves)
  auto load_code = [&](int cs, int hf, int q) {
    const int p = hf * S::QB + q;
    const uint8_t* src = bsrc[q] + (hf ? bsrc[S::QB + q] - bsrc[q] : 0);
    const int ko = 64 * cs + 16 * (lane >> 4);
    dma16(src + (ko + 16 <= K / 2 ? 64 * cs : -16 * (lane >> 4)),
          smem + S::C_OFF + (cs % 3) * S::CSLOT + (2 * S::QB * wave + p) * 1024);
  };
  // scale piece sp (64 columns) of scale stage t
  auto load_scale = [&](int t, int sp) {
    const int ko = 16 * t;
    dma16(ssrc + (size_t)mcol(64 * sp + lane) * (size_t)(K / 16) + (ko + 16 <= K / 16 ? ko : 0),
          smem + S::S_OFF + (t % 3) * S::SSLOT + 64 * sp * 16);
  };
  // the loads issued for K step kt (AHEAD steps ahead). E2M1: first, on two
  // wavefronts (even kt: 0, 1; odd kt: 2, 3), one scale piece of stage
  // (kt + 3) / 4; then A; then half (kt + 1) % 2 of code stage (kt + 1) / 2.
  // (Each stage is loaded after the stage three before it, same LDS slot, was
  // last read; the first pieces repeat stage 0, loaded before the loop.)
  auto issue = [&](int kt, int st) {
    uint8_t* As = smem + st * S::STAGE;
    if constexpr (WF == W_FP4) {
      if ((kt & 1) == (wave >> 1)) {
        const int sp = NSP == 8 ? 2 * ((kt + 3) & 3) + (wave & 1) : ((kt + 3) & 3);
        if (NSP == 8 || (wave & 1) == 0) load_scale((kt + 3) >> 2, sp);
      }
    }
#pragma unroll
    for (int q = 0; q < S::QA; ++q) dma16(asrc[q] + 64 * kt, As + ((S::BM / 4) * wave + 16 * q) * 64);
#pragma unroll
    for (int q = 0; q < S::QB; ++q) {
      if (WF == W_FP8)
        dma16(bsrc[q] + 64 * kt, As + S::A_STAGE + ((S::BN / 4) * wave + 16 * q) * 64);
      else
        load_code((kt + 1) >> 1, (kt + 1) & 1, q);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto bcol = [&](int j) -> int {
    if (GATE_UP) return (j < 2) ? 64 * wn + 32 * j : S::BN / 2 + 64 * wn + 32 * (j - 2);
    return 128 * wn + 32 * j;
  };
  const int l32 = lane & 31, kh = lane >> 5;
  const uint32_t lds0 = (uint32_t)(size_t)(lds_u8*)smem;
  const uint32_t rowb = (uint32_t)(size_t)(lds_u8*)rowdata;
  // A lane's 32 K values of a 64-deep step: bytes 0-15 of its operand belong
  // to the MFMA's first 32-value scale block, bytes 16-31 to the second, and
  // the two lane halves interleave in 16-value runs (measured), so lane half
  // kh takes K 16 kh .. +16 and 32 + 16 kh .. +16: each scale block is then 32
  // contiguous K values (two NVFP4 blocks), for A and B alike.
  uint32_t aoff[4][2], boff[4][2], soff[4];
  const uint32_t roff = rowb + 4 * (32 * wm + l32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 128 * wm + 32 * i + l32;
    aoff[i][0] = a_off(row, kh);
    aoff[i][1] = a_off(row, kh + 2);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = bcol(j) + l32;
    if (WF == W_FP8) {
      boff[j][0] = S::A_STAGE + a_off(c, kh);
      boff[j][1] = S::A_STAGE + a_off(c, kh + 2);
    } else {  // E2M1: run r (8 B = 16 codes) = 16 B chunk r of the K step
      boff[j][0] = (c >> 4) * 1024 + 16 * (c & 15) + 8 * kh;
      boff[j][1] = boff[j][0] + 256;
    }
    soff[j] = c * 16;
  }
  // One half of a K step: all four A fragments, the B codes of two column
  // tiles (j = 2h, 2h+1) and, for the down GEMM, the four rows' block scales
  // (one dword, byte i for row tile i). Raw read results stay separate
  // registers until their wait (they are the operands of the wait, so nothing
  // copies them while the reads are in flight).
  struct Half {
    u32x4 a[4][2];
    u32x4 b[2][2];     // E4M3: the two 16 B runs per column tile
    u32x2 q[2][2];     // E2M1: the two 8 B runs per column tile
    uint32_t sc[2];    // E2M1 block-scale dwords
    uint32_t as;       // down: E8M0 scales of the four rows
  };
  auto read_half = [&](Half& f, int st, int h, int kt) {
    const uint32_t base = lds0 + st * S::STAGE;
    // E2M1: chunks 2 (kt % 2), +1 of code stage kt / 2; scale bytes 4 (kt % 4) .. +3
    // of scale stage kt / 4
    const uint32_t cbase = lds0 + S::C_OFF + ((kt >> 1) % 3) * S::CSLOT + (kt & 1) * 512;
    const uint32_t sbase = lds0 + S::S_OFF + ((kt >> 2) % 3) * S::SSLOT + 4 * (kt & 3);
    if constexpr (WF == W_FP8) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * h + jj;
        f.b[jj][0] = lds_b128(base + boff[j][0]);
        f.b[jj][1] = lds_b128(base + boff[j][1]);
      }
    } else {
      // column tiles 2h and 2h + 1 are 32 columns (two 16-column blocks, 2 KB of
      // codes, 512 B of scales) apart; a column's second 8 B run is 256 B on
      const uint32_t cb = cbase + boff[2 * h][0], sb = sbase + soff[2 * h];
      f.q[0][0] = lds_b64o<0>(cb);
      f.q[0][1] = lds_b64o<256>(cb);
      f.sc[0] = lds_b32o<0>(sb);
      f.q[1][0] = lds_b64o<2048>(cb);
      f.q[1][1] = lds_b64o<2048 + 256>(cb);
      f.sc[1] = lds_b32o<512>(sb);
    }
    // rows 32 i + l32 of the A tile sit 2 KB apart at the same swizzled chunks
    const uint32_t a0 = base + aoff[0][0], a1 = base + aoff[0][1];
    f.a[0][0] = lds_b128o<0>(a0);
    f.a[0][1] = lds_b128o<0>(a1);
    f.a[1][0] = lds_b128o<2048>(a0);
    f.a[1][1] = lds_b128o<2048>(a1);
    f.a[2][0] = lds_b128o<4096>(a0);
    f.a[2][1] = lds_b128o<4096>(a1);
    f.a[3][0] = lds_b128o<6144>(a0);
    f.a[3][1] = lds_b128o<6144>(a1);
    if (!GATE_UP) f.as = lds_b32(roff + (kt >> 1) * S::BM);
  };
#define MOE_F8_WAIT_A(f, pending, ...)                                                        \
  asm volatile("s_waitcnt lgkmcnt(" #pending ")"                                              \
               : "+v"(f.a[0][0]), "+v"(f.a[0][1]), "+v"(f.a[1][0]), "+v"(f.a[1][1]),           \
                 "+v"(f.a[2][0]), "+v"(f.a[2][1]), "+v"(f.a[3][0]), "+v"(f.a[3][1]),           \
                 "+v"(f.as), __VA_ARGS__                                                       \
               :                                                                               \
               : "memory")
#define MOE_F8_WAIT_FP8(f, pending) \
  MOE_F8_WAIT_A(f, pending, "+v"(f.b[0][0]), "+v"(f.b[1][0]), "+v"(f.b[0][1]), "+v"(f.b[1][1]))
#define MOE_F8_WAIT_FP4(f, pending)                                                       \
  MOE_F8_WAIT_A(f, pending, "+v"(f.q[0][0]), "+v"(f.q[0][1]), "+v"(f.q[1][0]), "+v"(f.q[1][1]), \
                "+v"(f.sc[0]), "+v"(f.sc[1]))
  // reads per half: E4M3 weights 12 (gate/up) or 13 (down, with the row
  // scales); E2M1 weights 14 or 15 (at most 15 LDS reads are counted)
  auto wait_half = [&](Half& f) {
    if constexpr (WF == W_FP8) {
      if constexpr (GATE_UP)
        MOE_F8_WAIT_FP8(f, 12);
      else
        MOE_F8_WAIT_FP8(f, 13);
    } else {
      if constexpr (GATE_UP)
        MOE_F8_WAIT_FP4(f, 14);
      else
        MOE_F8_WAIT_FP4(f, 15);
    }
  };
  auto mfma_half = [&](const Half& f, int h) {
    i32x8 af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = i32x8{(int)f.a[i][0][0], (int)f.a[i][0][1], (int)f.a[i][0][2], (int)f.a[i][0][3],
                    (int)f.a[i][1][0], (int)f.a[i][1][1], (int)f.a[i][1][2], (int)f.a[i][1][3]};
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      i32x8 bf;
      int sb = 127;  // E8M0 scale of this lane's 32-deep K block of B
      if constexpr (WF == W_FP8) {
        bf = i32x8{(int)f.b[jj][0][0], (int)f.b[jj][0][1], (int)f.b[jj][0][2], (int)f.b[jj][0][3],
                   (int)f.b[jj][1][0], (int)f.b[jj][1][1], (int)f.b[jj][1][2], (int)f.b[jj][1][3]};
      } else {
        // run r (bytes 16 r .. of the operand) holds NVFP4 block kh + 2 r of the
        // step, in the MFMA's scale block r = K 32 r .. +32 (NVFP4 blocks 2 r,
        // 2 r + 1). Scale block r is shifted by 2^-s, s = (exponent field of
        // its larger E4M3 scale) - 12: every product e2m1 * s_blk * 2^-s stays
        // below 384 (never saturates) and the larger scale's nonzero products
        // are >= 16, whatever the scales' range. The shift goes into the
        // converter's power of two; this lane hands 2^s of scale block kh to
        // the MFMA (lane l: column l % 32, block l / 32).
        const uint32_t sc = f.sc[jj];
        const uint32_t s0 = sc & 0x7Fu, s1 = (sc >> 8) & 0x7Fu;  // magnitude codes order
        const uint32_t s2 = (sc >> 16) & 0x7Fu, s3 = (sc >> 24) & 0x7Fu;  // like values
        const uint32_t em[2] = {(s0 > s1 ? s0 : s1) >> 3, (s2 > s3 ? s2 : s3) >> 3};
        sb = (int)(115u + (kh ? em[1] : em[0]));
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint32_t c = (sc >> (8 * (kh + 2 * r))) & 0xFFu;  // NVFP4 block kh + 2 r
          const uint32_t ce = (c >> 3) & 15u, cm = c & 7u;
          const uint32_t normal = ce != 0u ? 1u : 0u;
          // 2^(e - 7) * 2^(12 - em): the block scale's power of two, shifted
          const float pb = __uint_as_float(((normal ? ce : 1u) + 132u - em[r]) << 23);
          const float fmr = (float)((normal << 3) | cm) * 0.125f;  // exact
          const float fm = __uint_as_float(__float_as_uint(fmr) | ((c & 0x80u) << 24));
          int32_t o0, o1, o2, o3;
          fp4_to_fp8(f.q[jj][r][0], pb, fm, o0, o1);
          fp4_to_fp8(f.q[jj][r][1], pb, fm, o2, o3);
          bf[4 * r] = o0;
          bf[4 * r + 1] = o1;
          bf[4 * r + 2] = o2;
          bf[4 * r + 3] = o3;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sa = GATE_UP ? 127 : (int)((f.as >> (8 * i)) & 0xFFu);
        acc[i][2 * h + jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            af[i], bf, acc[i][2 * h + jj], 0, 0, 0, sa, 0, sb);
      }
    }
  };

  // Pipeline as in the bf16 kernel, with NST stages and NST - 1 steps in flight.
  constexpr int AHEAD = S::NST - 1;
  const int nk = K / 64;
  if constexpr (WF == W_FP4) {  // code stage 0 and scale stage 0
#pragma unroll
    for (int p = 0; p < 2 * S::QB; ++p) load_code(0, p / S::QB, p % S::QB);
    for (int sp = wave; sp < NSP; sp += 4) load_scale(0, sp);
  }
  issue(0, 0);
  issue(nk > 1 ? 1 : nk - 1, 1);
  if constexpr (AHEAD == 3) issue(nk > 2 ? 2 : nk - 1, 2);
  vm_wait<(AHEAD - 1) * S::PER_STEP>();
  __builtin_amdgcn_s_barrier();
  Half f0, f1;
#pragma unroll
  for (int x = 0; x < 2; ++x) f0.sc[x] = f1.sc[x] = 0u;
  f0.as = f1.as = 0x7F7F7F7Fu;
  read_half(f0, 0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % S::NST;
    read_half(f1, st, 1, kt);
    wait_half(f0);
    mfma_half(f0, 0);
    vm_wait<(AHEAD - 2) * S::PER_STEP>();
    __builtin_amdgcn_s_barrier();
    issue(kt + AHEAD < nk ? kt + AHEAD : nk - 1, (kt + AHEAD) % S::NST);
    read_half(f0, (kt + 1) % S::NST, 0, kt + 1);
    wait_half(f1);
    mfma_half(f1, 1);
  }
  if constexpr (WF == W_FP8)
    MOE_F8_WAIT_FP8(f0, 0);
  else
    MOE_F8_WAIT_FP4(f0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef MOE_F8_WAIT_A
#undef MOE_F8_WAIT_FP8
#undef MOE_F8_WAIT_FP4
  __builtin_amdgcn_s_barrier();

  // ---- epilogue (strips reuse the pipeline's LDS; row data lies past it)
  const float gsc = WF == W_FP4 ? a.w_gscale[e] : 1.f;
  const float* chs = WF == W_FP8 ? static_cast<const float*>(a.w_scale) + (size_t)e * N : nullptr;
  auto tile_row = [&](int r) { return 8 * (r >> 2) + 4 * kh + (r & 3); };
  if (GATE_UP) {
    float sg[2], su[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sg[j] = WF == W_FP8 ? chs[mcol(bcol(j) + l32)] : gsc;
      su[j] = WF == W_FP8 ? chs[mcol(bcol(j + 2) + l32)] : gsc;
    }
    const float* xs = reinterpret_cast<const float*>(rowdata);
    uint16_t* strip = reinterpret_cast<uint16_t*>(smem + wave * 4096);  // 32 x 64 bf16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float rs = xs[(128 * wm + 32 * i + tile_row(r)) * (S::ROWB / 4)];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          strip[tile_row(r) * 64 + 32 * j + l32] = (uint16_t)f32_to_bf16_bits(
              silu(acc[i][j][r] * (rs * sg[j])) * (acc[i][j + 2][r] * (rs * su[j])));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = lane + 64 * t, rr = c >> 3, ch = c & 7;
        const int m = m0 + 128 * wm + 32 * i + rr;
        const int col = nt * (S::BN / 2) + 64 * wn + 8 * ch;
        const u32x4 v = *reinterpret_cast<const u32x4*>(strip + rr * 64 + 8 * ch);
        if (m < cnt && col < a.I)
          *reinterpret_cast<u32x4*>(a.h_out + (size_t)(r0 + m) * a.I + col) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else {
    float sd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sd[j] = WF == W_FP8 ? chs[mcol(bcol(j) + l32)] : gsc;
    float* strip = reinterpret_cast<float*>(smem + wave * 16384);  // 32 x 128 fp32
    const bool compact = a.y16 != nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) strip[tile_row(r) * 128 + 32 * j + l32] = acc[i][j][r] * sd[j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (compact) {  // compact rows: two 64-column scale blocks per strip row
        store_rows16<128>(strip, lane, m0 + 128 * wm + 32 * i, cnt, nt * S::BN + 128 * wn, N,
                          (size_t)r0, a.y16, a.y16_scale);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        continue;
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int c = lane + 64 * t, rr = c >> 5, ch = c & 31;
        const int m = m0 + 128 * wm + 32 * i + rr;
        const int col = nt * S::BN + 128 * wn + 4 * ch;
        const f32x4 v = *reinterpret_cast<const f32x4*>(strip + rr * 128 + 4 * ch);
        if (m < cnt && col < N) store_rows(a.y_out + (size_t)(r0 + m) * N + col, v);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// Activations -> E4M3 codes with one fp32 scale per token (amax / 448, 1 for a
// zero row); one workgroup per token, 8 values per lane per pass.
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t* __restrict__ x, int H,
                                                      uint8_t* __restrict__ xq,
                                                      float* __restrict__ xs) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint16_t* xr = x + (size_t)t * H;
  float m = 0.f;
  for (int c = 8 * tid; c < H; c += 2048) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(xr + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = fmaxf(m, fabsf(__uint_as_float(q[i] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(q[i] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (tid == 0) xs[t] = s;
  for (int c = 8 * tid; c < H; c += 2048) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(xr + c);
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float v0 = __uint_as_float(q[2 * h] << 16) / s;
      const float v1 = __uint_as_float(q[2 * h] & 0xFFFF0000u) / s;
      const float v2 = __uint_as_float(q[2 * h + 1] << 16) / s;
      const float v3 = __uint_as_float(q[2 * h + 1] & 0xFFFF0000u) / s;
      const int32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
      o[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, r, true);
    }
    *reinterpret_cast<uint2*>(xq + (size_t)t * H + c) = make_uint2(o[0], o[1]);
  }
}

// h (bf16) -> E4M3 codes with one E8M0 scale per row and 128-column block: the
// smallest 2^e with 448 * 2^e >= the block's amax (clamped to [-127, 127]; 0
// for a zero block). One wavefront per row; 16 lanes x 8 values per block.
__global__ __launch_bounds__(256) void quant_h_kernel(const uint16_t* __restrict__ h, int P, int I,
                                                      uint8_t* __restrict__ hq,
                                                      uint8_t* __restrict__ hs, int hs_stride) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= P) return;
  const uint16_t* hr = h + (size_t)row * I;
  for (int c0 = 0; c0 < I; c0 += 512) {
    const int c = c0 + 8 * lane;
    const bool ok = c < I;
    u32x4 q = u32x4{0u, 0u, 0u, 0u};
    if (ok) q = *reinterpret_cast<const u32x4*>(hr + c);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));  // within 16 lanes
    const uint32_t mb = __float_as_uint(m);
    const int ex = (int)(mb >> 23), man = (int)(mb & 0x7FFFFF);
    int eb;
    if (mb == 0u)
      eb = 0;
    else if (ex == 0)
      eb = -127;  // subnormal amax: far below the clamp
    else
      eb = (man <= 0x600000) ? ex - 127 - 8 : ex - 127 - 7;
    eb = eb < -127 ? -127 : (eb > 127 ? 127 : eb);
    // 2^-eb as fp32 (a normal number: eb <= 120 for any bf16 amax, and
    // eb = -127 gives 2^127); the scaled values are exact
    const float inv = __uint_as_float((uint32_t)(127 - eb) << 23);
    uint32_t o[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * hh] * inv, v[4 * hh + 1] * inv, 0, false);
      o[hh] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4 * hh + 2] * inv, v[4 * hh + 3] * inv, r, true);
    }
    if (ok) {
      *reinterpret_cast<uint2*>(hq + (size_t)row * I + c) = make_uint2(o[0], o[1]);
      if ((lane & 15) == 0) hs[(size_t)row * hs_stride + c / 128] = (uint8_t)(eb + 127);
    }
  }
}

}  // namespace

template <int WF, bool GATE_UP>
static hipError_t launch_q(const StreamGemmArgs& g, const int32_t* te, const int32_t* tm,
                           const int32_t* nt_p, int max_tiles, hipStream_t st) {
  using S = QShape<WF>;
  const int NT = GATE_UP ? (g.I + S::BN / 2 - 1) / (S::BN / 2) : (g.N + S::BN - 1) / S::BN;
  const long long items = (long long)max_tiles * NT;
  const unsigned grid = (unsigned)(((items + 7) / 8) * 8);
  if (grid == 0) return hipSuccess;
  tile_q_kernel<WF, GATE_UP><<<grid, 64 * S::NW, 0, st>>>(g, te, tm, nt_p, NT);
  return hipGetLastError();
}

template <int WF>
static hipError_t launch_q_all(const StreamGemmArgs& gu, const StreamGemmArgs& dn,
                               const int32_t* tile_e, const int32_t* tile_m0, const int32_t* counts,
                               int max_tiles, hipStream_t st) {
  hipError_t err = launch_q<WF, true>(gu, tile_e, tile_m0, counts, max_tiles, st);
  if (err == hipSuccess) err = launch_q<WF, false>(dn, tile_e, tile_m0, counts, max_tiles, st);
  return err;
}

template <int WF, bool GATE_UP, int WM>
static hipError_t launch_f8(const F8Args& f8, const StreamGemmArgs& g, const int32_t* te,
                            const int32_t* tm, const int32_t* nt_p, int max_tiles, hipStream_t st) {
  using S = F8Shape<WF, WM>;
  const int NT = GATE_UP ? (g.I + S::BN / 2 - 1) / (S::BN / 2) : (g.N + S::BN - 1) / S::BN;
  const long long items = (long long)max_tiles * NT;
  const unsigned grid = (unsigned)(((items + 7) / 8) * 8);
  if (grid == 0) return hipSuccess;
  tile_f8_kernel<WF, GATE_UP, WM><<<grid, 256, 0, st>>>(f8, g, te, tm, nt_p, NT);
  return hipGetLastError();
}

template <int WF>
static hipError_t launch_f8_all(const StreamGemmArgs& gu, const StreamGemmArgs& dn, int T, int P,
                                const F8Buffers& b, const int32_t* tile_e, const int32_t* tile_m0,
                                const int32_t* counts, int max_tiles, hipStream_t st) {
  quant_x_kernel<<<T, 256, 0, st>>>(gu.a, gu.K, b.xq, b.xs);
  hipError_t err = hipGetLastError();
  F8Args fg{b.xq, b.xs, nullptr, 0};
  if (err == hipSuccess) err = launch_f8<WF, true, 1>(fg, gu, tile_e, tile_m0, counts, max_tiles, st);
  if (err != hipSuccess) return err;
  quant_h_kernel<<<(P + 3) / 4, 256, 0, st>>>(gu.h_out, P, gu.I, b.hq, b.hs, b.hs_stride);
  err = hipGetLastError();
  F8Args fd{b.hq, nullptr, b.hs, b.hs_stride};
  if (err == hipSuccess) err = launch_f8<WF, false, 1>(fd, dn, tile_e, tile_m0, counts, max_tiles, st);
  return err;
}

hipError_t launch_expert_f8(int wfmt, const StreamGemmArgs& gu, const StreamGemmArgs& dn, int T,
                            int P, const F8Buffers& bufs, void* ws, hipStream_t st) {
  const int E = gu.E;
  if (wfmt != W_FP8 && wfmt != W_FP4) return hipErrorInvalidValue;
  // one table of 128-row tiles (128 x 512 tiles, as for the exact dequantisation)
  const int max_tiles = (P + 127) / 128 + E;
  int32_t* tile_e = static_cast<int32_t*>(ws);
  int32_t* tile_m0 = tile_e + max_tiles;
  int32_t* counts = tile_m0 + max_tiles;
  tile_table_kernel<<<1, 256, 0, st>>>(gu.offsets, E, 128, 0, tile_e, tile_m0, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (wfmt == W_FP8)
    return launch_f8_all<W_FP8>(gu, dn, T, P, bufs, tile_e, tile_m0, counts, max_tiles, st);
  return launch_f8_all<W_FP4>(gu, dn, T, P, bufs, tile_e, tile_m0, counts, max_tiles, st);
}

hipError_t launch_expert_tile_q(int wfmt, const StreamGemmArgs& gu, const StreamGemmArgs& dn, int P,
                                void* ws, hipStream_t st) {
  const int E = gu.E;
  int32_t* tile_e = static_cast<int32_t*>(ws);
  // one table of 128-row tiles, an expert's last of up to 160 (its tail of
  // <= 32 rows merged): at most P/128 + E of them
  const int max_tiles = (P + 127) / 128 + E;
  // the kernels address one expert's codes as a buffer
  if ((long long)gu.N * gu.K > 0x7FFFFFFFLL || (long long)dn.N * dn.K > 0x7FFFFFFFLL)
    return hipErrorInvalidValue;
  int32_t* tile_m0 = tile_e + max_tiles;
  int32_t* counts = tile_m0 + max_tiles;
  tile_table_kernel<<<1, 256, 0, st>>>(gu.offsets, E, 128, 32, tile_e, tile_m0, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (wfmt == W_FP8) return launch_q_all<W_FP8>(gu, dn, tile_e, tile_m0, counts, max_tiles, st);
  if (wfmt == W_FP4) return launch_q_all<W_FP4>(gu, dn, tile_e, tile_m0, counts, max_tiles, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
