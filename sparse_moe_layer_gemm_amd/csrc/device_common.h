// Device helpers shared by the gfx950 kernels: vector types, bf16 / fp16
// rounding, SiLU, expert-row stores and the weight-code converters.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- device helpers
// bf16 <-> fp32 (round to nearest, ties to even; inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Order-preserving map of a float onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Compact expert rows: the power-of-two exponent s that puts a block maximum
// m > 0 into [2^14, 2^15) after scaling by 2^-s (so fp16 rounding cannot
// overflow), clamped to the E8M0 byte range; 0 for an all-zero block.
__device__ __forceinline__ int rows16_exp(float m) {
  if (!(m > 0.f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(m);  // m = f * 2^e, f in [0.5, 1)
  const int s = e - 1 - 14;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
// Stores of the fp32 expert rows: written once and read once by the finalize
// step, long after, so they skip cache retention (nontemporal). Measured on
// gfx950 at decode sizes, this halves what the row stores add to the weight
// stream of the down projection.
__device__ __forceinline__ void store_rows(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store_rows(float* p, float v) { __builtin_nontemporal_store(v, p); }

// ---- weight-code converters (gfx950 hardware conversions)
typedef float f32x2 __attribute__((ext_vector_type(2)));
// E4M3 block scale -> (power of two, mantissa factor) as fp32, branch-free:
// normal codes give (2^(e-7), 1 + m/8), subnormal ones m * 2^-9 give
// (2^-6, m/8), zero gives a zero factor; the sign goes on the factor.
__device__ __forceinline__ void e4m3_split(uint32_t c, float& p2, float& fm) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const uint32_t normal = e != 0u ? 1u : 0u;
  p2 = __uint_as_float(((normal ? e : 1u) + 120u) << 23);
  const float f = (float)((normal << 3) | m) * 0.125f;  // exact
  fm = __uint_as_float(__float_as_uint(f) | ((c & 0x80u) << 24));
}
// Two E2M1 codes scaled by 2^e (converter) and the mantissa factor (fp32
// multiply) -> packed bf16: the products have at most 6 significant bits, so
// they and their bf16 upper halves are exact.
__device__ __forceinline__ uint32_t fp4_pair(f32x2 v, float fm) {
  return __builtin_amdgcn_perm(__float_as_uint(v.y * fm), __float_as_uint(v.x * fm), 0x07060302u);
}
// 8 E2M1 codes (one dword, even K in the low nibble) x block scale -> 8 bf16
__device__ __forceinline__ u32x4 fp4_frag(uint32_t d, float p2, float fm) {
  u32x4 r;
  r[0] = fp4_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, p2, 0), fm);
  r[1] = fp4_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, p2, 1), fm);
  r[2] = fp4_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, p2, 2), fm);
  r[3] = fp4_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, p2, 3), fm);
  return r;
}
// 8 E4M3 codes (two dwords) -> 8 bf16 (exact)
__device__ __forceinline__ u32x4 fp8_frag(uint32_t d0, uint32_t d1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
  return r;
}

}  // namespace moe
