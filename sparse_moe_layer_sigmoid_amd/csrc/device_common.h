// Device-side helpers shared by the libmoe kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bfloat16 bit pattern (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Unpack 8 bf16 held in a 16-byte word.
__device__ __forceinline__ void unpack_bf16x8(const u32x4& v, float f[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// float -> OCP E4M3FN code, round to nearest even, saturating to +/-448, NaN -> 0x7F|sign.
// The code's sign bit is the input's sign bit.  Written from the format's definition:
// below 2^-6 the spacing is 2^-9 (subnormals, and code 8 is the smallest normal, so
// rint(|v| * 2^9) is the code directly); above, keep 3 mantissa bits with RNE on the 20
// dropped bits.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  // branch-free: every lane takes both roundings and selects, so a wave never diverges
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  // normal range: round the 20 dropped mantissa bits to nearest even in the integer domain
  // (a carry moves into the exponent field), then rebias the exponent from 127 to 7
  const uint32_t qn = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  // below 2^-6: multiples of 2^-9, rounded to nearest even by the hardware
  const uint32_t qs = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  uint32_t q = a < 0x3c800000u ? qs : qn;
  q = a >= 0x43e00000u ? 0x7eu : q;  // |v| >= 448 (or inf): saturate
  q = a > 0x7f800000u ? 0x7fu : q;   // NaN
  return sign | q;
}

// 1/s refined by one Newton step from the hardware reciprocal (close to correctly rounded).
__device__ __forceinline__ float recip_refined(float s) {
  const float r = __builtin_amdgcn_rcpf(s);
  return fmaf(fmaf(-s, r, 1.0f), r, r);
}

// v / s from the refined reciprocal rs of s: the product, then one correction with the exact
// residual v - q s, which lands on the correctly rounded quotient in all but rare
// double-rounding cases.
__device__ __forceinline__ float quotient(float v, float s, float rs) {
  const float q0 = v * rs;
  return fmaf(fmaf(-q0, s, v), rs, q0);
}

// Power-of-two tile scale: the smallest k with amax <= 448 * 2^k, clamped to [-127, 127]
// (0 for an all-zero tile), read off amax's bits: for amax = 1.f * 2^E, 448 = 1.75 * 2^8, so
// k = E - 8 when the significand is <= 1.75 (fraction bits <= 0x600000), else E - 7.
// Subnormal amax (< 2^-126) lies far below 448 * 2^-127 and takes the clamp.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax) & 0x7fffffffu;
  const int e = (int)(u >> 23) - 127;
  const int k = e - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return u == 0 ? 0 : (u < 0x00800000u ? -127 : min(127, max(-127, k)));
}
// 2^k as a float for k in [-126, 127] (exact).
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Matrix-core wrappers (gfx950).
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x128 E4M3 x E4M3 -> f32 (format code 0 = E4M3 for both operands, no block scale).
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// The same with E8M0 block scales: each lane's operand rows (its 32 K values) are scaled by
// 2^(code - 127) of the low byte of sa (first operand) / sb (second operand).
__device__ __forceinline__ f32x4 mfma_fp8_e8m0(const i32x8& a, const i32x8& b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float max16(float v) {  // over the 16-lane group of this lane
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace moe
