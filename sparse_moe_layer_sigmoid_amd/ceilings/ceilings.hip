// Micro-benchmarks of the MI355X (gfx950) ceilings that the layer's kernels are measured
// against.  They are measurement code, not part of the layer: built into their own library
// (libmoe_ceilings.so) and driven by `bench.py --ceilings`.
//
//   moe_ceil_hbm_read  streaming read of a device buffer with 16-byte vector loads
//   moe_ceil_dma_read  streaming read with direct-to-LDS DMA (global_load_lds_dwordx4) in the
//                      grouped GEMM's weight pattern: blocks of 256 rows x 128 bytes, each wave
//                      instruction 8 rows x 128 bytes, a three-slot LDS ring, one vmcnt wait
//                      and one barrier per step, one workgroup per CU walking its row blocks
//   moe_ceil_dma_read_ring  the same streaming read with a ring of `slots` (2..5) 32 KB slots, so
//                      slots - 1 steps are in flight per CU (how deep a ring HBM streaming needs)
//   moe_ceil_dma_resident  the same step pattern (256 rows x 128 bytes per step, 8 rows x 128 B
//                      per wave instruction, three-slot ring) over a working set chosen to sit in
//                      one cache level: workgroup b reads row block b % n_blocks over and over,
//                      `steps` K steps of its rows (wrapping around the row length); mode 0
//                      moves the data with direct-to-LDS DMA, mode 1 with 16-byte vector loads
//                      into registers.  A few row blocks shared by every workgroup stay in the
//                      L2; one row block per workgroup of a size the XCD's L2 cannot hold, but
//                      the Infinity Cache can, is served from there.  Per-CU rate from the
//                      workgroups' s_memtime cycles, chip rate from the launch time.
//   moe_ceil_lds_read  LDS read bandwidth with ds_read_b128 (width 16) or ds_read_b64 (8),
//                      one 8-wave workgroup per CU, conflict-free addresses; iters reads per
//                      lane (a multiple of 16)
//   moe_ceil_mfma      matrix-core rate from registers: kind 0 = bf16 16x16x32, 1 = E4M3
//                      16x16x128, 2 = E4M3 16x16x128 from zero with each result scaled and
//                      added into an fp32 accumulator (4 FMAs per product, the promotion of the
//                      E4M3 GEMM); 8 waves per workgroup (two per SIMD, as in the GEMM)
//   moe_ceil_valu      fp32 FMA rate (v_fma_f32: packed FP32 is not used by this library)
//
// Every call: grid workgroups on `stream`; each thread writes one word of `sink`
// (sink_words >= grid x threads per workgroup, so nothing is optimised away); the timed
// calls write each workgroup's s_memtime cycle count into cycles[grid] (device, u64).
// Returns 0, or -1 on a bad argument (nothing launched), or -2 when the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace {

constexpr int kRowsPerBlock = 256;  // one weight block of the GEMM: 256 rows x 128 bytes
constexpr int kStep = kRowsPerBlock * 128;

#define CEIL_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ p, size_t n, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 a = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 v0 = p[i], v1 = p[i + stride], v2 = p[i + 2 * stride], v3 = p[i + 3 * stride];
    a ^= v0 ^ v1 ^ v2 ^ v3;
  }
  for (; i < n; i += stride) a ^= p[i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = a[0] ^ a[1] ^ a[2] ^ a[3];
}

// 8 waves; wave w issues the 4 instructions q = 4w .. 4w+3 of a step (rows 8q .. 8q+7 of the
// 256-row block, lane l: row 8q + l/8, bytes 16 (l%8) of the step's 128-byte column slice).
__global__ __launch_bounds__(512) void dma_read_kernel(const uint8_t* __restrict__ buf, int n_rb, int row_bytes,
                                                       uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[kStep];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[kStep];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[kStep];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int steps_per_rb = row_bytes / 128;
  const int n_my = blockIdx.x < n_rb ? (n_rb - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int64_t n = (int64_t)n_my * steps_per_rb;
  auto issue = [&](int64_t g) {
    const int64_t rb = blockIdx.x + (g / steps_per_rb) * gridDim.x;
    const int k = (int)(g % steps_per_rb);
    const int s = (int)(g % 3);
    uint8_t* st = s == 0 ? slot0 : (s == 1 ? slot1 : slot2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = wave * 4 + j;
      const int64_t row = rb * kRowsPerBlock + q * 8 + (lane >> 3);
      const uint8_t* src = buf + row * row_bytes + k * 128 + (lane & 7) * 16;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(st + q * 1024), 16, 0, 0);
    }
  };
  if (n > 0) issue(0);
  if (n > 1) issue(1);
  for (int64_t g = 0; g < n; ++g) {
    if (g + 1 < n) CEIL_WAIT_VM(4); else CEIL_WAIT_VM(0);  // step g has landed
    __builtin_amdgcn_s_barrier();                          // ... for every wave: slot (g+2)%3 is free
    if (g + 2 < n) issue(g + 2);
  }
  sink[(size_t)blockIdx.x * 512 + threadIdx.x] = (uint32_t)n;
}

// dma_read_kernel's walk with an NS-slot ring: NS - 1 steps in flight, one wait and one barrier
// per step (a slot is refilled one step after it was waited for, once every wave is past it)
template <int NS>
__global__ __launch_bounds__(512) void dma_ring_kernel(const uint8_t* __restrict__ buf, int n_rb, int row_bytes,
                                                       uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t slot[NS][kStep];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int steps_per_rb = row_bytes / 128;
  const int n_my = blockIdx.x < n_rb ? (n_rb - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int64_t n = (int64_t)n_my * steps_per_rb;
  auto issue = [&](int64_t g) {
    const int64_t rb = blockIdx.x + (g / steps_per_rb) * gridDim.x;
    const int k = (int)(g % steps_per_rb);
    uint8_t* st = slot[g % NS];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = wave * 4 + j;
      const int64_t row = rb * kRowsPerBlock + q * 8 + (lane >> 3);
      const uint8_t* src = buf + row * row_bytes + k * 128 + (lane & 7) * 16;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(st + q * 1024), 16, 0, 0);
    }
  };
  for (int64_t g = 0; g < NS - 1 && g < n; ++g) issue(g);
  for (int64_t g = 0; g < n; ++g) {
    // step g has landed: the batches of the min(NS - 2, n - 1 - g) later steps may still be in flight
    const int64_t later = n - 1 - g < NS - 2 ? n - 1 - g : NS - 2;
    if (later >= 3) CEIL_WAIT_VM(12);
    else if (later == 2) CEIL_WAIT_VM(8);
    else if (later == 1) CEIL_WAIT_VM(4);
    else CEIL_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();  // every wave is past step g - 1: its slot takes step g + NS - 1
    if (g + NS - 1 < n) issue(g + NS - 1);
  }
  sink[(size_t)blockIdx.x * 512 + threadIdx.x] = (uint32_t)n;
}

template <int MODE>
__global__ __launch_bounds__(512) void dma_resident_kernel(const uint8_t* __restrict__ buf, int n_blocks, int row_bytes,
                                                           int steps, uint64_t* cycles, uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t slot[3][kStep];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int steps_per_row = row_bytes / 128;
  const uint8_t* base = buf + (int64_t)(blockIdx.x % n_blocks) * kRowsPerBlock * row_bytes + (lane & 7) * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 r[3][4];
  // instruction j of wave w at step g: rows 8q .. 8q + 7 (q = 4w + j), the step's 128-byte slice
  auto issue = [&](int g, auto slot_c) {
    constexpr int s = decltype(slot_c)::value;
    const int k = g % steps_per_row;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = wave * 4 + j;
      const uint8_t* src = base + (int64_t)(q * 8 + (lane >> 3)) * row_bytes + k * 128;
      if (MODE == 0)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(&slot[s][q * 1024]), 16, 0, 0);
      else
        r[s][j] = *(const u32x4*)src;
    }
  };
  auto step = [&](int g, auto slot_c) {
    constexpr int s = decltype(slot_c)::value;
    CEIL_WAIT_VM(4);  // step g has landed (the 4 instructions of step g + 1 may still be in flight)
    if (MODE == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= r[s][j];
    }
    __builtin_amdgcn_s_barrier();  // every wave is past step g - 1: its slot takes step g + 2
    issue(g + 2, std::integral_constant<int, (s + 2) % 3>());
  };
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  issue(0, std::integral_constant<int, 0>());
  issue(1, std::integral_constant<int, 1>());
  for (int g = 0; g < steps; g += 3) {
    step(g, std::integral_constant<int, 0>());
    step(g + 1, std::integral_constant<int, 1>());
    step(g + 2, std::integral_constant<int, 2>());
  }
  CEIL_WAIT_VM(0);  // the two batches issued past the last step
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (MODE == 1) {
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= r[s][j];
  } else {
    acc[0] ^= slot[0][threadIdx.x];
  }
  sink[(size_t)blockIdx.x * 512 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

template <int WIDTH>
__global__ __launch_bounds__(512) void lds_read_kernel(int iters, uint64_t* cycles, uint32_t* sink) {
  // 96 KB, so that one workgroup holds a CU
  __shared__ __attribute__((aligned(16))) u32x4 lds[6144];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 6144; i += 512) lds[i] = u32x4{(uint32_t)i, (uint32_t)i * 3u, 7u, (uint32_t)i ^ 5u};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint32_t a = 0;
  if constexpr (WIDTH == 16) {
    const u32x4* base = lds + wave * 512 + lane;  // a wave's 1 KB rows, 4096 entries in use
    u32x4 v = {0u, 0u, 0u, 0u};
    for (int it = 0; it < iters; it += 8) {
      int off = 0;
      asm volatile("" : "+v"(off));  // opaque offset: the reads cannot be hoisted out of the loop
#pragma unroll
      for (int u = 0; u < 8; ++u) v ^= base[off + u * 64];
    }
    a = v[0] ^ v[1] ^ v[2] ^ v[3];
  } else {
    const u32x2* base = reinterpret_cast<const u32x2*>(lds) + wave * 1024 + lane;
    u32x2 v = {0u, 0u};
    for (int it = 0; it < iters; it += 16) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        int off = u * 64;
        asm volatile("" : "+v"(off));  // one opaque offset per read: no pairing into ds_read2
        v ^= base[off];
      }
    }
    a = v[0] ^ v[1];
  }
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  sink[(size_t)blockIdx.x * 512 + tid] = a;
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

template <int KIND>
__global__ __launch_bounds__(512) void mfma_kernel(int iters, uint64_t* cycles, uint32_t* sink) {
  const int tid = threadIdx.x;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if constexpr (KIND == 0) {
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(float)((tid + e) & 7);
      b[e] = (__bf16)(float)((tid * 3 + e) & 3);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = moe::mfma_bf16(a, b, acc[j]);
    }
  } else {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x38383838 ^ ((tid + e) & 0x03030303);  // E4M3 values near 1
      b[e] = 0x30303030 ^ ((tid * 5 + e) & 0x03030303);
    }
    if constexpr (KIND == 1) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = moe::mfma_fp8(a, b, acc[j]);
      }
    } else {
      const float s = 1.0f + (float)(tid & 7) * 0x1p-20f;
      for (int it = 0; it < iters; ++it) {
        f32x4 pq[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          asm volatile("" : "+v"(a));  // opaque operand: no product is hoisted out of the loop or merged
          pq[j] = moe::mfma_fp8(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(pq[j][r], s, acc[j][r]);
      }
    }
  }
  __syncthreads();  // the workgroup's time, not wave 0's (a SIMD's older wave may finish first)
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float f = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[(size_t)blockIdx.x * 512 + tid] = __float_as_uint(f);
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

__global__ __launch_bounds__(512) void valu_kernel(int iters, uint64_t* cycles, uint32_t* sink) {
  const int tid = threadIdx.x;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (float)(tid + j) * 1e-3f;
  const float m = 0.999f, c = 1e-4f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fmaf(v[j], m, c);
  }
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float f = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f += v[j];
  sink[(size_t)blockIdx.x * 512 + tid] = __float_as_uint(f);
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -2; }

}  // namespace

extern "C" {

int moe_ceil_hbm_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, int grid,
                      hipStream_t stream) {
  if (!buf || !sink || bytes % 16 || ((uintptr_t)buf & 15) || grid < 1 || sink_words < (size_t)grid * 256)
    return -1;
  hbm_read_kernel<<<grid, 256, 0, stream>>>(static_cast<const u32x4*>(buf), bytes / 16, sink);
  return launched();
}

// buf holds rows x row_bytes bytes; rows % 256 == 0, row_bytes % 128 == 0.
int moe_ceil_dma_read(const void* buf, int64_t rows, int row_bytes, uint32_t* sink, size_t sink_words, int grid,
                      hipStream_t stream) {
  if (!buf || !sink || rows < kRowsPerBlock || rows % kRowsPerBlock || row_bytes < 128 || row_bytes % 128 ||
      ((uintptr_t)buf & 15) || grid < 1 || rows / kRowsPerBlock > INT32_MAX || sink_words < (size_t)grid * 512)
    return -1;
  dma_read_kernel<<<grid, 512, 0, stream>>>(static_cast<const uint8_t*>(buf), (int)(rows / kRowsPerBlock),
                                            row_bytes, sink);
  return launched();
}

// as moe_ceil_dma_read, with `slots` (2..5) ring slots
int moe_ceil_dma_read_ring(int slots, const void* buf, int64_t rows, int row_bytes, uint32_t* sink, size_t sink_words,
                           int grid, hipStream_t stream) {
  if (slots < 2 || slots > 5 || !buf || !sink || rows < kRowsPerBlock || rows % kRowsPerBlock || row_bytes < 128 ||
      row_bytes % 128 || ((uintptr_t)buf & 15) || grid < 1 || rows / kRowsPerBlock > INT32_MAX ||
      sink_words < (size_t)grid * 512)
    return -1;
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  const int n_rb = (int)(rows / kRowsPerBlock);
  if (slots == 2) dma_ring_kernel<2><<<grid, 512, 0, stream>>>(b, n_rb, row_bytes, sink);
  else if (slots == 3) dma_ring_kernel<3><<<grid, 512, 0, stream>>>(b, n_rb, row_bytes, sink);
  else if (slots == 4) dma_ring_kernel<4><<<grid, 512, 0, stream>>>(b, n_rb, row_bytes, sink);
  else dma_ring_kernel<5><<<grid, 512, 0, stream>>>(b, n_rb, row_bytes, sink);
  return launched();
}

// buf holds n_blocks x 256 rows x row_bytes bytes; row_bytes % 128 == 0; steps a positive
// multiple of 3; cycles[grid] (u64) receives each workgroup's cycle count.
int moe_ceil_dma_resident(int mode, const void* buf, int n_blocks, int row_bytes, int steps, uint64_t* cycles,
                          uint32_t* sink, size_t sink_words, int grid, hipStream_t stream) {
  if ((mode != 0 && mode != 1) || !buf || !cycles || !sink || n_blocks < 1 || row_bytes < 128 || row_bytes % 128 ||
      steps < 3 || steps % 3 || ((uintptr_t)buf & 15) || grid < 1 || sink_words < (size_t)grid * 512)
    return -1;
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  if (mode == 0) dma_resident_kernel<0><<<grid, 512, 0, stream>>>(b, n_blocks, row_bytes, steps, cycles, sink);
  else dma_resident_kernel<1><<<grid, 512, 0, stream>>>(b, n_blocks, row_bytes, steps, cycles, sink);
  return launched();
}

int moe_ceil_lds_read(int width, int iters, uint64_t* cycles, uint32_t* sink, size_t sink_words, int grid,
                      hipStream_t stream) {
  if ((width != 8 && width != 16) || iters < 16 || iters % 16 || !cycles || !sink || grid < 1 || sink_words < (size_t)grid * 512)
    return -1;
  if (width == 16) lds_read_kernel<16><<<grid, 512, 0, stream>>>(iters, cycles, sink);
  else lds_read_kernel<8><<<grid, 512, 0, stream>>>(iters, cycles, sink);
  return launched();
}

int moe_ceil_mfma(int kind, int iters, uint64_t* cycles, uint32_t* sink, size_t sink_words, int grid,
                  hipStream_t stream) {
  if (kind < 0 || kind > 2 || iters < 1 || !cycles || !sink || grid < 1 || sink_words < (size_t)grid * 512)
    return -1;
  if (kind == 0) mfma_kernel<0><<<grid, 512, 0, stream>>>(iters, cycles, sink);
  else if (kind == 1) mfma_kernel<1><<<grid, 512, 0, stream>>>(iters, cycles, sink);
  else mfma_kernel<2><<<grid, 512, 0, stream>>>(iters, cycles, sink);
  return launched();
}

int moe_ceil_valu(int iters, uint64_t* cycles, uint32_t* sink, size_t sink_words, int grid, hipStream_t stream) {
  if (iters < 1 || !cycles || !sink || grid < 1 || sink_words < (size_t)grid * 512) return -1;
  valu_kernel<<<grid, 512, 0, stream>>>(iters, cycles, sink);
  return launched();
}

}  // extern "C"
