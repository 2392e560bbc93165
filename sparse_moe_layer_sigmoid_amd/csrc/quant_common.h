// The E4M3 tile encoding shared by the quantisation kernels (fp8_quant_1x128 / 128x128) and the
// fused transpose-and-quantise of the backward pass, so both produce the same codes.
#pragma once

#include "device_common.h"

namespace moe {

// Eight values to E4M3 codes (4 per dword, little-endian) with the tile scale s: q = RNE(v / s),
// an IEEE division per element.
__device__ __forceinline__ u32x2 encode8(const float f[8], float s) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(f[i] / s) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(f[4 + i] / s) << (8 * i);
  return u32x2{lo, hi};
}

}  // namespace moe
