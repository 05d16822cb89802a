// Device pieces shared by the tiled expert kernels (many rows per expert):
// tile shapes, LDS fill and fragment reads, the 32x32x16 MFMA, the A tile
// swizzle, the compact-row epilogue and the M-tile table.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TBK = 32, NSTAGE = 4;
constexpr int TBM = 256;  // rows of the large tile (tile table sizing, router)

// Workgroup tile shapes. WM wavefronts along M: WM = 2 gives 256 x 256 tiles,
// WM = 1 gives 128 x 512 tiles (for experts, or expert tails, of <= 128 rows).
// NW wavefronts per workgroup: with 4, each computes 128 x 128 (one per
// SIMD); with 8, each computes 128 x 64 and two share a SIMD, so that one can
// issue MFMAs while the other waits on its loads or the barrier.
template <int WM, int NW = 4>
struct TileShape {
  static constexpr int BM = 128 * WM, BN = 512 / WM;
  static constexpr int WN = NW / WM;            // wavefronts along N
  static constexpr int WCOLS = BN / WN;         // columns per wavefront (128 or 64)
  static constexpr int JT = WCOLS / 32;         // 32-column MFMA tiles per wavefront
  static constexpr int A_STAGE = BM * TBK * 2;  // BM rows x 64 B
  static constexpr int B_STAGE = TBK * BN * 2;  // 32 rows x 2*BN B
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS = NSTAGE * STAGE;    // 128 KB / 160 KB (also the epilogue staging)
  static constexpr int QA = BM / 16 / NW;       // 1 KB (16-row) A loads per wavefront per K step
  static constexpr int QB = BN / 16 / NW;       // 1 KB B loads per wavefront per K step
  static constexpr int RPI = 512 / BN;          // B rows per load
  static constexpr int ARW = BM / NW;           // A rows each wavefront loads
  static constexpr int BRW = TBK / NW;          // B rows each wavefront loads
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Direct global -> LDS load: lane l's 16 bytes land at lds + 16 * l.
__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
// LDS reads the compiler does not see (their results are only valid after an
// explicit lgkmcnt wait that takes them as operands).
__device__ __forceinline__ u32x4 lds_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
__device__ __forceinline__ u32x2 lds_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// v_mfma_f32_32x32x16_bf16: lane l supplies A row l%32 / B column l%32 with K
// block l/32 (8 values); the result lane l holds column l%32, rows
// 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// A rows are 64 B (4 granules); granule g of row r sits at g ^ ((r >> 2) & 3), so
// the 16 consecutive rows of one fragment read cover all 16 bank groups.
__device__ __forceinline__ int a_off(int row, int g) { return row * 64 + ((g ^ ((row >> 2) & 3)) << 4); }
// B rows are 512 B (32 granules). A half-wave of transpose reads touches 4
// consecutive K rows at two adjacent 32-byte column chunks; XOR-ing the
// granule index with 4 * (row % 4) puts those 8 reads in distinct banks.
__device__ __forceinline__ int b_swz(int row) { return (row & 3) << 2; }

// Maximum over each aligned group of 8 lanes, in every lane of the group
// (DPP: swap neighbours, swap pairs, then mirror within the half row).
__device__ __forceinline__ float max8_lanes(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  return v;
}

// Compact rows from a wavefront's LDS strip of 32 rows x SW fp32 columns
// (SW = 64 or 128: one or two 64-column scale blocks per row), the strip's
// row rr being output row row0 + rr and its column 0 output column col0. Eight
// adjacent lanes hold one block's 8 chunks of 8 values, so the block maximum
// is three DPP steps; each chunk leaves as one 16-byte store of fp16 values,
// each block's scale as one byte.
template <int SW>
__device__ __forceinline__ void store_rows16(const float* strip, int lane, int row0, int cnt,
                                             int col0, int N, size_t r0, uint16_t* __restrict__ y16,
                                             uint8_t* __restrict__ y16_scale) {
  constexpr int CPR = SW / 8;  // 8-value chunks per strip row
  const int nb = N / 64;
#pragma unroll
  for (int t = 0; t < SW / 16; ++t) {  // 32 rows x CPR chunks over 64 lanes
    const int c = lane + 64 * t, rr = c / CPR, ch = c % CPR;
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(strip + rr * SW + 8 * ch);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(strip + rr * SW + 8 * ch + 4);
    float mx = fmaxf(fmaxf(fmaxf(fabsf(v0[0]), fabsf(v0[1])), fmaxf(fabsf(v0[2]), fabsf(v0[3]))),
                     fmaxf(fmaxf(fabsf(v1[0]), fabsf(v1[1])), fmaxf(fabsf(v1[2]), fabsf(v1[3]))));
    mx = max8_lanes(mx);
    const int sx = rows16_exp(mx);
    const float inv = __builtin_ldexpf(1.0f, -sx);
    u32x4 pk;
    pk[0] = f32_to_f16_bits(v0[0] * inv) | (f32_to_f16_bits(v0[1] * inv) << 16);
    pk[1] = f32_to_f16_bits(v0[2] * inv) | (f32_to_f16_bits(v0[3] * inv) << 16);
    pk[2] = f32_to_f16_bits(v1[0] * inv) | (f32_to_f16_bits(v1[1] * inv) << 16);
    pk[3] = f32_to_f16_bits(v1[2] * inv) | (f32_to_f16_bits(v1[3] * inv) << 16);
    const int m = row0 + rr;
    const int col = col0 + 8 * ch;
    if (m < cnt && col < N) {
      __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(y16 + (r0 + m) * (size_t)N + col));
      if ((ch & 7) == 0) y16_scale[(r0 + m) * (size_t)nb + col / 64] = (uint8_t)(sx + 127);
    }
  }
}

// M-tile table, in expert order: ceil(rows / bm) tiles of bm rows per expert.
// With merge > 0 an expert's last tile also takes a tail of up to `merge`
// rows (tiles of bm rows, the last of up to bm + merge).
__global__ __launch_bounds__(256) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                         int E, int bm, int merge,
                                                         int32_t* __restrict__ tile_e,
                                                         int32_t* __restrict__ tile_m0,
                                                         int32_t* __restrict__ n_tiles) {
  __shared__ int cnt[256];
  const int e = threadIdx.x;
  const int rows = (e < E) ? offsets[e + 1] - offsets[e] : 0;
  int c = (rows - merge + bm - 1) / bm;
  if (rows > 0 && c < 1) c = 1;
  if (rows <= 0) c = 0;
  cnt[e] = c;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {  // inclusive scan
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

__device__ __forceinline__ u32x2 lds_b64(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
__device__ __forceinline__ uint32_t lds_b32(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
__device__ __forceinline__ uint32_t lds_byte(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_u8 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
// dword direct load: lane l's 4 bytes land at lds + 4 * l
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}

}  // namespace
}  // namespace moe
