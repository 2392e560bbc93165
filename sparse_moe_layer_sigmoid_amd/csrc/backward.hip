// The layer's backward pass: the element-wise and gather kernels between its GEMMs (which run on
// moe_grouped_gemm), written from the chain rule of the forward definition ("DeepSeek-V3
// Technical Report" (wiki summary), "DeepSeekMoE と補助損失なしの負荷分散": gates are the
// selected affinities normalised to sum to one, the bias only selects; "FP8 混合精度訓練": a
// training step runs the layer's Fprop, Dgrad and Wgrad).
//
//  * moe_combine_backward: one workgroup per token.  From d_out and the routed expert outputs
//    it forms the down projection's input gradient rows (gate * d_out at each pair's sorted
//    row, d_out itself at the token's shared row), the gate gradients dg_k = <d_out, y_k>
//    (fp32, fixed order) and from them the router logit gradients of the selected experts:
//    with S = sum_k s_k, du_k = s_k (1 - s_k) (dg_k - sum_j g_j dg_j) / S.
//  * moe_swiglu_backward: da = dh c silu'(a), dc = dh silu(a), silu'(a) = sig(a)(1 + a(1 - sig(a))),
//    four elements per lane, HBM-bound.
//  * moe_segment_transpose: row segments of a row-major matrix (optionally gathered) become
//    column blocks of its transpose, each padded with zero columns to a given start (or, with
//    a segment stride, separate zero-padded [cols, width] blocks), so each expert's
//    weight-gradient GEMM reduces over its own rows with K-contiguous operands, and equal-width
//    blocks let one grouped GEMM cover every expert.  128 x 128 tiles, each lane an 8 x 8 block
//    transposed in registers; 16-byte loads and stores.
//  * moe_segment_transpose_fp8: the same into equal-width blocks, quantised to E4M3 on the way
//    ("FP8 混合精度訓練": Wgrad runs in FP8 on transposed operands, and the report's "考察" asks
//    for the transposition and the quantisation to be fused) with the 1x128 scales along each
//    block row or one scale per 128x128 block, the codes those quantisers give on the bf16
//    transpose.
//  * moe_router_wgrad: dW_r[e] = sum over e's sorted rows r of du_row[r] * x[token(r)], one
//    workgroup per (expert, 2048 columns), rows in order (deterministic).
#include "abi_common.h"
#include "device_common.h"
#include "quant_common.h"

namespace moe {
namespace {

constexpr int kMaxBwdK = 32;

__global__ __launch_bounds__(256) void combine_backward_kernel(
    const uint16_t* __restrict__ d_out, const uint16_t* __restrict__ y, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ scores, const int32_t* __restrict__ pair_pos, int T,
    int K, int d, int N, uint16_t* __restrict__ dy, float* __restrict__ du, float* __restrict__ du_row,
    uint8_t* __restrict__ dyq, float* __restrict__ dys) {
  __shared__ int s_p[kMaxBwdK];
  __shared__ float s_g[kMaxBwdK];
  __shared__ float s_part[kMaxBwdK][4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < K) {
    s_p[tid] = pair_pos[(int64_t)t * K + tid];
    s_g[tid] = gate[(int64_t)t * K + tid];
  }
  __syncthreads();
  float dot[kMaxBwdK];
#pragma unroll
  for (int k = 0; k < kMaxBwdK; ++k) dot[k] = 0.f;
  const int nc = d / 8;
  const uint16_t* orow = d_out + (int64_t)t * d;
  // with dyq: each dy row also as E4M3 with 1x128 scales, quantised from its bf16 values as
  // fp8_quant_1x128 does; the 16 lanes of a 1x128 tile are 16 consecutive chunks (d % 128 == 0,
  // so whole 16-lane groups share the loop's trip count)
  auto quant_row = [&](int64_t row, int c, const u32x4& bits) {
    float q[8];
    unpack_bf16x8(bits, q);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(q[i]));
    amax = max16(amax);
    const float s = (amax == 0.f) ? 1.0f : amax / 448.0f;
    *(u32x2*)(dyq + row * d + c * 8) = encode8(q, s);
    if ((c & 15) == 0) dys[row * (d / 128) + c / 16] = s;
  };
  for (int c = tid; c < nc; c += 256) {
    const u32x4 ov = *(const u32x4*)(orow + c * 8);
    *(u32x4*)(dy + ((int64_t)T * K + t) * d + c * 8) = ov;  // the shared expert's row: d_out itself
    if (dyq) quant_row((int64_t)T * K + t, c, ov);
    float f[8];
    unpack_bf16x8(ov, f);
#pragma unroll
    for (int k = 0; k < kMaxBwdK; ++k) {
      if (k < K && s_p[k] >= 0) {  // pairs skipped by the permutation (p < 0) carry nothing
        const int64_t p = s_p[k];
        float yv[8];
        unpack_bf16x8(*(const u32x4*)(y + p * d + c * 8), yv);
        float acc = dot[k];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(f[i], yv[i], acc);
        dot[k] = acc;
        const float g = s_g[k];
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_rne(g * f[2 * i]) | (f32_to_bf16_rne(g * f[2 * i + 1]) << 16);
        *(u32x4*)(dy + p * d + c * 8) = o;
        if (dyq) quant_row(p, c, o);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxBwdK; ++k) {
    if (k < K) {
      float v = dot[k];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
      if (lane == 0) s_part[k][wave] = v;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane k < K: gate gradient, selected affinity; then the two sums over the K lanes
    float dg = 0.f, s = 0.f, g = 0.f;
    const int e = lane < K ? idx[(int64_t)t * K + lane] : -1;
    const bool valid = lane < K && s_p[lane] >= 0 && e >= 0 && e < N;
    if (valid) {
      dg = ((s_part[lane][0] + s_part[lane][1]) + s_part[lane][2]) + s_part[lane][3];
      s = scores[(int64_t)t * N + e];
      g = s_g[lane];
    }
    float S = s, gd = g * dg;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      S += __shfl_xor(S, o, kWave);
      gd += __shfl_xor(gd, o, kWave);
    }
    if (lane < K) {
      const float u = valid ? (dg - gd) / S * (s * (1.0f - s)) : 0.f;
      du[(int64_t)t * K + lane] = u;
      if (valid) du_row[s_p[lane]] = u;
    }
  }
}

__global__ __launch_bounds__(256) void swiglu_backward_kernel(const float* __restrict__ ac,
                                                              const float* __restrict__ dh, int64_t n4, int I,
                                                              uint16_t* __restrict__ dac, uint8_t* __restrict__ dacq,
                                                              float* __restrict__ dacs) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // quad of h elements
  if (q >= n4) return;
  const int qi = I / 4;
  const int64_t r = q / qi;
  const int i = (int)(q - r * qi) * 4;
  const f32x4 a = *(const f32x4*)(ac + r * 2 * I + i);
  const f32x4 c = *(const f32x4*)(ac + r * 2 * I + I + i);
  const f32x4 g = *(const f32x4*)(dh + r * I + i);
  float da[4], dc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a[e]));
    dc[e] = g[e] * (a[e] * sg);
    da[e] = g[e] * c[e] * (sg * (1.0f + a[e] * (1.0f - sg)));
  }
  const u32x2 pa = u32x2{f32_to_bf16_rne(da[0]) | (f32_to_bf16_rne(da[1]) << 16),
                         f32_to_bf16_rne(da[2]) | (f32_to_bf16_rne(da[3]) << 16)};
  const u32x2 pc = u32x2{f32_to_bf16_rne(dc[0]) | (f32_to_bf16_rne(dc[1]) << 16),
                         f32_to_bf16_rne(dc[2]) | (f32_to_bf16_rne(dc[3]) << 16)};
  *(u32x2*)(dac + r * 2 * I + i) = pa;
  *(u32x2*)(dac + r * 2 * I + I + i) = pc;
  if (dacq) {
    // the 1x128 E4M3 quantisation of the stored bf16 da | dc, as fp8_quant_1x128 does it: the 32
    // lanes of a tile are 32 consecutive quads of one row (I % 128 == 0, so whole 32-lane groups
    // share the early exit above)
    const u32x2 pk[2] = {pa, pc};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        f[2 * e] = bf16_to_f32(pk[h][e] & 0xffffu);
        f[2 * e + 1] = bf16_to_f32(pk[h][e] >> 16);
      }
      float amax = fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3])));
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
      const float s = (amax == 0.f) ? 1.0f : amax / 448.0f;
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) w |= f32_to_e4m3(f[e] / s) << (8 * e);
      const int col = h * I + i;
      *(uint32_t*)(dacq + r * 2 * I + col) = w;
      if ((i & 127) == 0) dacs[r * (2 * I / 128) + col / 128] = s;
    }
  }
}

// A workgroup transposes 128 output columns (source rows) x 128 channels; wave w covers the
// column half w & 1 and the channel half w >> 1 (64 x 64), lane (jb, ch) = (lane & 7, lane >> 3)
// the 8 output columns 8 jb .. 8 jb + 7 and the 8 channels 8 ch .. 8 ch + 7 of it: it loads 8
// source rows of 16 bytes, transposes the 8 x 8 block of bf16 in registers and stores 8 channel
// rows of 8 values.  A load instruction of the wave covers 8 rows x 128 contiguous bytes, a store
// instruction 8 channel rows x 128 (bf16) or 64 (E4M3) contiguous bytes; no LDS for the data.

// Source row of output column j in segment block g (block start `start`), or -1 for a padding
// column.
__device__ __forceinline__ int column_source(int j, int g, int start, const int32_t* __restrict__ seg,
                                             const int32_t* __restrict__ gather) {
  const int r0 = seg[g], i = j - start;
  if (i < 0 || i >= seg[g + 1] - r0) return -1;
  return gather ? gather[r0 + i] : r0 + i;
}

// v[r] = 8 bf16 channels of source row r  ->  o[i] = 8 bf16 output columns of channel i.
__device__ __forceinline__ void transpose8x8(const u32x4 (&v)[8], u32x4 (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int w = i >> 1, sh = (i & 1) * 16;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[i][k] = ((v[2 * k][w] >> sh) & 0xffffu) | (((v[2 * k + 1][w] >> sh) & 0xffffu) << 16);
  }
}

__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ src, int64_t lds, const int (&srow)[8], int c,
                                          bool cvalid, u32x4 (&v)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    v[r] = u32x4{0u, 0u, 0u, 0u};
    if (cvalid && srow[r] >= 0) v[r] = *(const u32x4*)(src + (int64_t)srow[r] * lds + c);
  }
}

// bf16 output, any column blocks (dst_cols multiples of 8).
__global__ __launch_bounds__(256) void segment_transpose_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                                const int32_t* __restrict__ gather,
                                                                const int32_t* __restrict__ seg,
                                                                const int32_t* __restrict__ col, int G, int C,
                                                                int total, uint16_t* __restrict__ dst, int64_t ldd,
                                                                int64_t seg_stride) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int jb = lane & 7, ch = lane >> 3;
  const int j = blockIdx.x * 128 + (w & 1) * 64 + jb * 8;
  const int c = blockIdx.y * 128 + (w >> 1) * 64 + ch * 8;
  if (j >= total) return;
  int lo = 0, hi = G;  // the segment block holding column j: the largest g with col[g] <= j
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (col[mid] <= j) lo = mid;
    else hi = mid;
  }
  // the lane's 8 columns: a block boundary inside them moves the later ones to the next block
  // (blocked output needs block starts that are multiples of 8, so it never happens there)
  int srow[8];
  int g = lo;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    while (g + 1 < G && col[g + 1] <= j + r) ++g;
    srow[r] = column_source(j + r, g, col[g], seg, gather);
  }
  u32x4 v[8], o[8];
  load_rows(src, lds, srow, c, c < C, v);
  transpose8x8(v, o);
  const int64_t at = seg_stride > 0 ? (int64_t)lo * seg_stride + (j - col[lo]) : (int64_t)j;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (c + i < C) *(u32x4*)(dst + at + (int64_t)(c + i) * ldd) = o[i];
}

// E4M3 output in equal-width blocks [G][C][width] with the scales of fp8_quant_1x128 applied
// along each block row (BLOCK = false: scale [G * C][width / 128]) or of fp8_quant_128x128 per
// block (BLOCK = true: scale [G][C / 128][width / 128]), the same rule and divisions as those
// kernels, so the codes equal quantising the bf16 transpose.  The workgroup's 128 columns are
// one 128-column tile of one block (width % 128 == 0), its 128 channels one 128-row block.
template <bool BLOCK>
__global__ __launch_bounds__(256) void segment_transpose_fp8_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                                    const int32_t* __restrict__ gather,
                                                                    const int32_t* __restrict__ seg, int C, int width,
                                                                    uint8_t* __restrict__ q, float* __restrict__ scale) {
  // BLOCK: the four waves' maxima; else each channel row's maxima over the two column halves
  __shared__ float red[BLOCK ? 4 : 2 * 128];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int jb = lane & 7, ch = lane >> 3, half = w & 1;
  const int tiles = width / 128;
  const int g = blockIdx.x / tiles, tile = blockIdx.x - g * tiles;
  const int jl = tile * 128 + half * 64 + jb * 8;  // column within the block
  const int cl = (w >> 1) * 64 + ch * 8;            // channel within the workgroup's 128
  const int c = blockIdx.y * 128 + cl;
  int srow[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) srow[r] = column_source(jl + r, g, 0, seg, gather);
  u32x4 v[8], o[8];
  load_rows(src, lds, srow, c, true, v);
  transpose8x8(v, o);
  float f[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) unpack_bf16x8(o[i], f[i]);
  uint8_t* qb = q + ((int64_t)g * C + c) * width + jl;
  if constexpr (BLOCK) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(f[i][k]));
    amax = wave_max(amax);
    if (lane == 0) red[w] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = (amax == 0.f) ? 1.0f : amax / 448.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x2*)(qb + (int64_t)i * width) = encode8(f[i], s);
    if (threadIdx.x == 0) scale[((int64_t)g * (C / 128) + blockIdx.y) * tiles + tile] = s;
  } else {
    float amax[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float m = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[i][k]));
#pragma unroll
      for (int o2 = 1; o2 < 8; o2 <<= 1) m = fmaxf(m, __shfl_xor(m, o2, kWave));  // the 8 lanes of the half row
      amax[i] = m;
      if (jb == 0) red[(cl + i) * 2 + half] = m;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float m = fmaxf(amax[i], red[(cl + i) * 2 + (half ^ 1)]);  // with the other column half
      const float s = (m == 0.f) ? 1.0f : m / 448.0f;
      *(u32x2*)(qb + (int64_t)i * width) = encode8(f[i], s);
      if (jb == 0 && half == 0) scale[((int64_t)g * C + c + i) * tiles + tile] = s;
    }
  }
}

__global__ __launch_bounds__(256) void router_wgrad_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ sorted_token,
                                                           const int32_t* __restrict__ offs,
                                                           const float* __restrict__ du_row, int d,
                                                           float* __restrict__ dw) {
  const int e = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= d) return;
  const int r0 = offs[e], r1 = offs[e + 1];
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int r = r0; r < r1; ++r) {
    const float w = du_row[r];
    float f[8];
    unpack_bf16x8(*(const u32x4*)(x + (int64_t)sorted_token[r] * d + c), f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, f[i], acc[i]);
  }
  float* o = dw + (int64_t)e * d + c;
  *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_combine_backward(const uint16_t* d_out, const uint16_t* y_routed, const int32_t* topk_idx,
                                           const float* topk_gate, const float* scores, const int32_t* pair_pos,
                                           int T, int top_k, int d, int n_experts, uint16_t* dy, float* du,
                                           float* du_row, uint8_t* dy_q, float* dy_scale, hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(T == 0 || (d_out && y_routed && topk_idx && topk_gate && scores && pair_pos && dy && du && du_row),
              MOE_ERR_NULL, "moe_combine_backward: a required pointer is NULL");
  MOE_REQUIRE(!dy_q == !dy_scale, MOE_ERR_NULL, "moe_combine_backward: dy_q and dy_scale go together");
  MOE_REQUIRE(T >= 0 && top_k >= 1 && top_k <= kMaxBwdK && top_k <= n_experts && d >= 8 && d % 8 == 0 &&
                  (!dy_q || d % 128 == 0),
              MOE_ERR_SHAPE,
              "moe_combine_backward: T=%d top_k=%d (1..%d) d=%d (a multiple of 8; of 128 with dy_q) n_experts=%d", T,
              top_k, kMaxBwdK, d, n_experts);
  MOE_REQUIRE(aligned16(d_out) && aligned16(y_routed) && aligned16(dy) && ((uintptr_t)dy_q & 7u) == 0 &&
                  ((uintptr_t)dy_scale & 3u) == 0,
              MOE_ERR_ALIGN, "moe_combine_backward: d_out, y_routed and dy must be 16-byte, dy_q 8-byte aligned");
  if (T > 0)
    combine_backward_kernel<<<T, 256, 0, stream>>>(d_out, y_routed, topk_idx, topk_gate, scores, pair_pos, T, top_k, d,
                                                   n_experts, dy, du, du_row, dy_q, dy_scale);
  return check_launch("moe_combine_backward");
}

extern "C" moe_status moe_swiglu_backward(const float* ac, const float* dh, int64_t rows, int inter, uint16_t* dac,
                                          uint8_t* dac_q, float* dac_scale, hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(rows == 0 || (ac && dh && dac), MOE_ERR_NULL, "moe_swiglu_backward: a required pointer is NULL");
  MOE_REQUIRE(!dac_q == !dac_scale, MOE_ERR_NULL, "moe_swiglu_backward: dac_q and dac_scale go together");
  MOE_REQUIRE(rows >= 0 && inter >= 4 && inter % 4 == 0 && (!dac_q || inter % 128 == 0), MOE_ERR_SHAPE,
              "moe_swiglu_backward: rows=%lld inter=%d (a positive multiple of 4; of 128 with dac_q)", (long long)rows,
              inter);
  MOE_REQUIRE(aligned16(ac) && aligned16(dh) && ((uintptr_t)dac & 7u) == 0 && ((uintptr_t)dac_q & 3u) == 0 &&
                  ((uintptr_t)dac_scale & 3u) == 0,
              MOE_ERR_ALIGN, "moe_swiglu_backward: ac and dh must be 16-byte, dac 8-byte, dac_q 4-byte aligned");
  const int64_t n4 = rows * (inter / 4);
  if (n4 > 0) {
    const int64_t grid = (n4 + 255) / 256;
    MOE_REQUIRE(grid < (int64_t)1 << 31, MOE_ERR_SHAPE, "moe_swiglu_backward: too many rows");
    swiglu_backward_kernel<<<(unsigned)grid, 256, 0, stream>>>(ac, dh, n4, inter, dac, dac_q, dac_scale);
  }
  return check_launch("moe_swiglu_backward");
}

extern "C" moe_status moe_segment_transpose(const uint16_t* src, int64_t ld_src, const int32_t* src_rows,
                                            const int32_t* seg_offsets, const int32_t* dst_cols, int n_segments,
                                            int cols, int total_cols, uint16_t* dst, int64_t ld_dst,
                                            int64_t seg_stride, hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(seg_offsets && dst_cols && (total_cols == 0 || (src && dst)), MOE_ERR_NULL,
              "moe_segment_transpose: a required pointer is NULL");
  MOE_REQUIRE(n_segments >= 1 && cols >= 8 && cols % 8 == 0 && total_cols >= 0 && total_cols % 8 == 0, MOE_ERR_SHAPE,
              "moe_segment_transpose: n_segments=%d cols=%d total_cols=%d (cols, total_cols multiples of 8)",
              n_segments, cols, total_cols);
  MOE_REQUIRE(seg_stride >= 0 && seg_stride % 8 == 0, MOE_ERR_ALIGN, "moe_segment_transpose: seg_stride=%lld",
              (long long)seg_stride);
  MOE_REQUIRE(ld_src >= cols && ld_src % 8 == 0 && ld_dst % 8 == 0 && (seg_stride > 0 || ld_dst >= total_cols) &&
                  aligned16(src) && aligned16(dst),
              MOE_ERR_ALIGN, "moe_segment_transpose: ld_src=%lld ld_dst=%lld must keep rows 16-byte aligned",
              (long long)ld_src, (long long)ld_dst);
  if (total_cols > 0) {
    const dim3 grid((total_cols + 127) / 128, (cols + 127) / 128);
    segment_transpose_kernel<<<grid, 256, 0, stream>>>(src, ld_src, src_rows, seg_offsets, dst_cols, n_segments, cols,
                                                       total_cols, dst, ld_dst, seg_stride);
  }
  return check_launch("moe_segment_transpose");
}

extern "C" moe_status moe_segment_transpose_fp8(const uint16_t* src, int64_t ld_src, const int32_t* src_rows,
                                                const int32_t* seg_offsets, int n_segments, int cols, int width,
                                                int block_scales, uint8_t* q, float* scale, hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(src && seg_offsets && q && scale, MOE_ERR_NULL, "moe_segment_transpose_fp8: a required pointer is NULL");
  MOE_REQUIRE(n_segments >= 1 && cols >= 128 && cols % 128 == 0 && cols / 128 <= 65535 && width >= 128 &&
                  width % 128 == 0 && (block_scales == 0 || block_scales == 1) &&
                  (int64_t)n_segments * (width / 128) < ((int64_t)1 << 31),
              MOE_ERR_SHAPE,
              "moe_segment_transpose_fp8: n_segments=%d cols=%d width=%d (multiples of 128) block_scales=%d (0 or 1)",
              n_segments, cols, width, block_scales);
  MOE_REQUIRE(ld_src >= cols && ld_src % 8 == 0 && aligned16(src) && ((uintptr_t)q & 7u) == 0 &&
                  ((uintptr_t)scale & 3u) == 0,
              MOE_ERR_ALIGN,
              "moe_segment_transpose_fp8: ld_src=%lld (>= cols, a multiple of 8), src 16-byte, q 8-byte and scale "
              "4-byte aligned",
              (long long)ld_src);
  const dim3 grid((unsigned)((int64_t)n_segments * (width / 128)), cols / 128);
  if (block_scales)
    segment_transpose_fp8_kernel<true><<<grid, 256, 0, stream>>>(src, ld_src, src_rows, seg_offsets, cols, width, q,
                                                                 scale);
  else
    segment_transpose_fp8_kernel<false><<<grid, 256, 0, stream>>>(src, ld_src, src_rows, seg_offsets, cols, width, q,
                                                                  scale);
  return check_launch("moe_segment_transpose_fp8");
}

extern "C" moe_status moe_router_wgrad(const uint16_t* x, const int32_t* sorted_token, const int32_t* expert_offsets,
                                       const float* du_row, int n_experts, int d, float* dw_router,
                                       hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(x && sorted_token && expert_offsets && du_row && dw_router, MOE_ERR_NULL,
              "moe_router_wgrad: a required pointer is NULL");
  MOE_REQUIRE(n_experts >= 1 && n_experts <= 65535 && d >= 8 && d % 8 == 0, MOE_ERR_SHAPE,
              "moe_router_wgrad: n_experts=%d d=%d (a multiple of 8)", n_experts, d);
  MOE_REQUIRE(aligned16(x) && aligned16(dw_router), MOE_ERR_ALIGN, "moe_router_wgrad: x and dw_router must be 16-byte aligned");
  const dim3 grid(n_experts, (d / 8 + 255) / 256);
  router_wgrad_kernel<<<grid, 256, 0, stream>>>(x, sorted_token, expert_offsets, du_row, d, dw_router);
  return check_launch("moe_router_wgrad");
}
