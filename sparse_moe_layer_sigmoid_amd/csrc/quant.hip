// fp8_quant_1x128 / fp8_quant_128x128: online E4M3 quantisation with fine-grained scales.
// "DeepSeek-V3 Technical Report" (wiki summary), "FP8 混合精度訓練": activations are scaled
// per 1x128 tile and weights per 128x128 block ("細粒度量子化"), the scale coming from the
// current max |value| of the tile or block ("オンライン量子化"), all stored as E4M3
// ("E4M3 統一").  Rule: s = fl32(amax / 448) (s = 1 for an all-zero tile), q = RNE(x / s)
// saturating at +/-448, both divisions IEEE-rounded so the codes are reproducible bit for bit.
//
// The *_e8m0 variants use a power-of-two scale per tile instead ("Vol.25 DeepSeek-V3の技術と
// その影響", "学習と推論の課題と解決策": a tile's values can share one exponent; the report's
// "考察" asks for tile / block scaling inside the matrix unit, which the gfx950 block-scaled
// MFMA provides): the smallest 2^k with amax / 2^k <= 448, k in [-127, 127] (0 for an
// all-zero tile), stored as the E8M0 code k + 127; x / 2^k is an exact product, so only the
// E4M3 rounding remains.
//
// Both kernels are HBM-bound streaming passes: 16-byte loads of 8 bf16 per lane, the amax
// reduced with lane shuffles (16 lanes per 1x128 tile) or shuffles + LDS (128x128 block).
#include "abi_common.h"
#include "device_common.h"
#include "quant_common.h"

namespace moe {
namespace {

// The same with a power-of-two scale: exact products by 2^-k.
__device__ __forceinline__ u32x2 encode8_pow2(const float f[8], float inv) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(f[i] * inv) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(f[4 + i] * inv) << (8 * i);
  return u32x2{lo, hi};
}

// 256 threads = 16 tiles of 1x128; lane group of 16 handles one tile, 8 values per lane.
// E8: power-of-two scales stored as E8M0 codes (uint8), else f32 scales.
template <bool E8>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const uint16_t* __restrict__ x,
                                                          int64_t n_tiles, int tiles_per_row,
                                                          int64_t ldx, uint8_t* __restrict__ q,
                                                          void* __restrict__ scale) {
  const int64_t tile = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (tile >= n_tiles) return;  // whole 16-lane groups leave together
  const int sub = threadIdx.x & 15;
  const int64_t r = tile / tiles_per_row;
  const int c = (int)(tile - r * tiles_per_row);
  const u32x4 v = *(const u32x4*)(x + r * ldx + (int64_t)c * 128 + sub * 8);
  float f[8];
  unpack_bf16x8(v, f);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = max16(amax);
  const int64_t cols = (int64_t)tiles_per_row * 128;
  if constexpr (E8) {
    const int k = e8m0_exponent(amax);
    *(u32x2*)(q + r * cols + (int64_t)c * 128 + sub * 8) = encode8_pow2(f, pow2f(-k));
    if (sub == 0) static_cast<uint8_t*>(scale)[tile] = (uint8_t)(k + 127);
  } else {
    const float s = (amax == 0.f) ? 1.0f : amax / 448.0f;
    *(u32x2*)(q + r * cols + (int64_t)c * 128 + sub * 8) = encode8(f, s);
    if (sub == 0) static_cast<float*>(scale)[tile] = s;
  }
}

// One workgroup per 128x128 block: thread t covers columns 8*(t%16)..+7 of rows t/16 + 16 j.
template <bool E8>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const uint16_t* __restrict__ w,
                                                            int n, int k,
                                                            uint8_t* __restrict__ q,
                                                            void* __restrict__ scale) {
  __shared__ float red[4];
  const int nbk = k / 128, nbn = n / 128;
  const int64_t blk = blockIdx.x;
  const int64_t mat = blk / ((int64_t)nbn * nbk);
  const int rem = (int)(blk - mat * nbn * nbk);
  const int bn = rem / nbk, bk = rem - bn * nbk;
  const int tid = threadIdx.x, c8 = (tid & 15) * 8, r0 = tid >> 4;
  const uint16_t* base = w + (mat * n + (int64_t)bn * 128) * k + (int64_t)bk * 128 + c8;
  float f[8][8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 v = *(const u32x4*)(base + (int64_t)(r0 + 16 * j) * k);
    unpack_bf16x8(v, f[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[j][i]));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  uint8_t* qb = q + (mat * n + (int64_t)bn * 128) * k + (int64_t)bk * 128 + c8;
  if constexpr (E8) {
    const int e = e8m0_exponent(amax);
    const float inv = pow2f(-e);
#pragma unroll
    for (int j = 0; j < 8; ++j) *(u32x2*)(qb + (int64_t)(r0 + 16 * j) * k) = encode8_pow2(f[j], inv);
    if (tid == 0) static_cast<uint8_t*>(scale)[blk] = (uint8_t)(e + 127);
  } else {
    const float s = (amax == 0.f) ? 1.0f : amax / 448.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) *(u32x2*)(qb + (int64_t)(r0 + 16 * j) * k) = encode8(f[j], s);
    if (tid == 0) static_cast<float*>(scale)[blk] = s;
  }
}

template <bool E8>
moe_status quant_1x128(const char* fn, const uint16_t* x, int rows, int cols, int64_t ldx, uint8_t* q, void* scale,
                       hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(rows == 0 || (x && q && scale), MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  MOE_REQUIRE(rows >= 0 && cols >= 128 && cols % 128 == 0, MOE_ERR_SHAPE,
              "%s: rows=%d cols=%d (cols must be a positive multiple of 128)", fn, rows, cols);
  MOE_REQUIRE(ldx >= cols && ldx % 8 == 0, MOE_ERR_ALIGN, "%s: ldx=%lld must be >= cols and a multiple of 8", fn,
              (long long)ldx);
  MOE_REQUIRE(aligned16(x) && ((uintptr_t)q & 7u) == 0, MOE_ERR_ALIGN, "%s: x must be 16-byte and q 8-byte aligned", fn);
  const int tpr = cols / 128;
  const int64_t n_tiles = (int64_t)rows * tpr;
  if (n_tiles > 0) {
    const int64_t grid = (n_tiles + 15) / 16;
    MOE_REQUIRE(grid < (int64_t)1 << 31, MOE_ERR_SHAPE, "%s: too many tiles", fn);
    quant_1x128_kernel<E8><<<(unsigned)grid, 256, 0, stream>>>(x, n_tiles, tpr, ldx, q, scale);
  }
  return check_launch(fn);
}

template <bool E8>
moe_status quant_128x128(const char* fn, const uint16_t* w, int n_mats, int n, int k, uint8_t* q, void* scale,
                         hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(w && q && scale, MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  MOE_REQUIRE(n_mats >= 0 && n >= 128 && k >= 128 && n % 128 == 0 && k % 128 == 0, MOE_ERR_SHAPE,
              "%s: n_mats=%d n=%d k=%d (n, k positive multiples of 128)", fn, n_mats, n, k);
  MOE_REQUIRE(aligned16(w) && ((uintptr_t)q & 7u) == 0, MOE_ERR_ALIGN, "%s: w must be 16-byte and q 8-byte aligned", fn);
  const int64_t blocks = (int64_t)n_mats * (n / 128) * (k / 128);
  MOE_REQUIRE(blocks < (int64_t)1 << 31, MOE_ERR_SHAPE, "%s: too many blocks", fn);
  if (blocks > 0) quant_128x128_kernel<E8><<<(unsigned)blocks, 256, 0, stream>>>(w, n, k, q, scale);
  return check_launch(fn);
}

// E4M3 code -> float (exact): E = 0 is M * 2^-9, else (1 + M/8) * 2^(E-7), rebuilt as fp32 bits.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 15u, m = c & 7u;
  const float sub = (float)m * (1.0f / 512.0f);
  const float v = e == 0 ? sub : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(v) | s);
}

// q * s per 1x128 tile, stored RNE bf16: 8 codes per lane.
__global__ __launch_bounds__(256) void dequant_1x128_kernel(const uint8_t* __restrict__ q, const float* __restrict__ scale,
                                                            int64_t n8, int cols, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t e0 = i * 8;
  const int64_t r = e0 / cols;
  const int c = (int)(e0 - r * cols);
  const float s = scale[r * (cols / 128) + c / 128];
  const u32x2 w = *(const u32x2*)(q + e0);
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t word = k < 2 ? w[0] : w[1];
    const int sh = (k & 1) * 16;
    const float lo = e4m3_to_f32((word >> sh) & 255u) * s, hi = e4m3_to_f32((word >> (sh + 8)) & 255u) * s;
    o[k] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
  }
  *(u32x4*)(out + e0) = o;
}

}  // namespace
}  // namespace moe

extern "C" moe_status fp8_quant_1x128(const uint16_t* x, int rows, int cols, int64_t ldx,
                                      uint8_t* q, float* scale, hipStream_t stream) {
  return moe::quant_1x128<false>("fp8_quant_1x128", x, rows, cols, ldx, q, scale, stream);
}

extern "C" moe_status fp8_quant_128x128(const uint16_t* w, int n_mats, int n, int k, uint8_t* q,
                                        float* scale, hipStream_t stream) {
  return moe::quant_128x128<false>("fp8_quant_128x128", w, n_mats, n, k, q, scale, stream);
}

extern "C" moe_status fp8_quant_1x128_e8m0(const uint16_t* x, int rows, int cols, int64_t ldx,
                                           uint8_t* q, uint8_t* scale, hipStream_t stream) {
  return moe::quant_1x128<true>("fp8_quant_1x128_e8m0", x, rows, cols, ldx, q, scale, stream);
}

extern "C" moe_status fp8_quant_128x128_e8m0(const uint16_t* w, int n_mats, int n, int k, uint8_t* q,
                                             uint8_t* scale, hipStream_t stream) {
  return moe::quant_128x128<true>("fp8_quant_128x128_e8m0", w, n_mats, n, k, q, scale, stream);
}

extern "C" moe_status fp8_dequant_1x128(const uint8_t* q, const float* scale, int rows, int cols, uint16_t* out,
                                        hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(rows == 0 || (q && scale && out), MOE_ERR_NULL, "fp8_dequant_1x128: a required pointer is NULL");
  MOE_REQUIRE(rows >= 0 && cols >= 128 && cols % 128 == 0, MOE_ERR_SHAPE, "fp8_dequant_1x128: rows=%d cols=%d", rows, cols);
  MOE_REQUIRE(((uintptr_t)q & 7u) == 0 && aligned16(out), MOE_ERR_ALIGN,
              "fp8_dequant_1x128: q must be 8-byte and out 16-byte aligned");
  const int64_t n8 = (int64_t)rows * cols / 8;
  if (n8 > 0) {
    const int64_t grid = (n8 + 255) / 256;
    MOE_REQUIRE(grid < (int64_t)1 << 31, MOE_ERR_SHAPE, "fp8_dequant_1x128: too many rows");
    dequant_1x128_kernel<<<(unsigned)grid, 256, 0, stream>>>(q, scale, n8, cols, out);
  }
  return check_launch("fp8_dequant_1x128");
}
