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
//    blocks let one grouped GEMM cover every expert.  64 x 64 tiles through LDS; both the loads
//    and the stores are 16-byte and coalesced.
//  * moe_router_wgrad: dW_r[e] = sum over e's sorted rows r of du_row[r] * x[token(r)], one
//    workgroup per (expert, 2048 columns), rows in order (deterministic).
#include "abi_common.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kMaxBwdK = 32;

__global__ __launch_bounds__(256) void combine_backward_kernel(
    const uint16_t* __restrict__ d_out, const uint16_t* __restrict__ y, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ scores, const int32_t* __restrict__ pair_pos, int T,
    int K, int d, int N, uint16_t* __restrict__ dy, float* __restrict__ du, float* __restrict__ du_row) {
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
  for (int c = tid; c < nc; c += 256) {
    const u32x4 ov = *(const u32x4*)(orow + c * 8);
    *(u32x4*)(dy + ((int64_t)T * K + t) * d + c * 8) = ov;  // the shared expert's row: d_out itself
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
                                                              uint16_t* __restrict__ dac) {
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
  *(u32x2*)(dac + r * 2 * I + i) = u32x2{f32_to_bf16_rne(da[0]) | (f32_to_bf16_rne(da[1]) << 16),
                                          f32_to_bf16_rne(da[2]) | (f32_to_bf16_rne(da[3]) << 16)};
  *(u32x2*)(dac + r * 2 * I + I + i) = u32x2{f32_to_bf16_rne(dc[0]) | (f32_to_bf16_rne(dc[1]) << 16),
                                              f32_to_bf16_rne(dc[2]) | (f32_to_bf16_rne(dc[3]) << 16)};
}

// Output column j of the transpose: source row of segment g = the segment whose padded column
// block holds j, or -1 for a padding column.
__device__ __forceinline__ int transpose_source(int j, const int32_t* __restrict__ seg, const int32_t* __restrict__ col,
                                                int G, const int32_t* __restrict__ gather, int* g_out) {
  int lo = 0, hi = G;  // largest g with col[g] <= j
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (col[mid] <= j) lo = mid;
    else hi = mid;
  }
  *g_out = lo;
  const int local = j - col[lo];
  if (local < 0 || local >= seg[lo + 1] - seg[lo]) return -1;
  const int r = seg[lo] + local;
  return gather ? gather[r] : r;
}

// 64 output columns x 64 channels per workgroup.  Loads: row (output column) jl, 16-byte chunk
// ch of its 64 channels; stores: channel row cl, 16-byte chunk of 8 output columns.
__global__ __launch_bounds__(256) void segment_transpose_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                                const int32_t* __restrict__ gather,
                                                                const int32_t* __restrict__ seg,
                                                                const int32_t* __restrict__ col, int G, int C,
                                                                int total, uint16_t* __restrict__ dst, int64_t ldd,
                                                                int64_t seg_stride) {
  __shared__ uint16_t tile[64][64 + 8];
  const int j0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + 256 * h;
    const int jl = e >> 3, ch = e & 7;
    const int j = j0 + jl;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < total && c0 + ch * 8 < C) {
      int g;
      const int s = transpose_source(j, seg, col, G, gather, &g);
      if (s >= 0) v = *(const u32x4*)(src + (int64_t)s * lds + c0 + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[jl][ch * 8 + 2 * i] = (uint16_t)(v[i] & 0xffffu);
      tile[jl][ch * 8 + 2 * i + 1] = (uint16_t)(v[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + 256 * h;
    const int cl = e >> 3, jc = e & 7;
    const int c = c0 + cl, j = j0 + jc * 8;
    if (c < C && j < total) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (uint32_t)tile[jc * 8 + 2 * i][cl] | ((uint32_t)tile[jc * 8 + 2 * i + 1][cl] << 16);
      int64_t at = (int64_t)c * ldd + j;
      if (seg_stride > 0) {  // blocked: segment g's block at g * seg_stride, columns from its start
        int lo = 0, hi = G;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (col[mid] <= j) lo = mid;
          else hi = mid;
        }
        at = (int64_t)lo * seg_stride + (int64_t)c * ldd + (j - col[lo]);
      }
      *(u32x4*)(dst + at) = o;
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
                                           float* du_row, hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(T == 0 || (d_out && y_routed && topk_idx && topk_gate && scores && pair_pos && dy && du && du_row),
              MOE_ERR_NULL, "moe_combine_backward: a required pointer is NULL");
  MOE_REQUIRE(T >= 0 && top_k >= 1 && top_k <= kMaxBwdK && top_k <= n_experts && d >= 8 && d % 8 == 0, MOE_ERR_SHAPE,
              "moe_combine_backward: T=%d top_k=%d (1..%d) d=%d (a multiple of 8) n_experts=%d", T, top_k, kMaxBwdK,
              d, n_experts);
  MOE_REQUIRE(aligned16(d_out) && aligned16(y_routed) && aligned16(dy), MOE_ERR_ALIGN,
              "moe_combine_backward: d_out, y_routed and dy must be 16-byte aligned");
  if (T > 0)
    combine_backward_kernel<<<T, 256, 0, stream>>>(d_out, y_routed, topk_idx, topk_gate, scores, pair_pos, T, top_k, d,
                                                   n_experts, dy, du, du_row);
  return check_launch("moe_combine_backward");
}

extern "C" moe_status moe_swiglu_backward(const float* ac, const float* dh, int64_t rows, int inter, uint16_t* dac,
                                          hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(rows == 0 || (ac && dh && dac), MOE_ERR_NULL, "moe_swiglu_backward: a required pointer is NULL");
  MOE_REQUIRE(rows >= 0 && inter >= 4 && inter % 4 == 0, MOE_ERR_SHAPE,
              "moe_swiglu_backward: rows=%lld inter=%d (a positive multiple of 4)", (long long)rows, inter);
  MOE_REQUIRE(aligned16(ac) && aligned16(dh) && ((uintptr_t)dac & 7u) == 0, MOE_ERR_ALIGN,
              "moe_swiglu_backward: ac and dh must be 16-byte, dac 8-byte aligned");
  const int64_t n4 = rows * (inter / 4);
  if (n4 > 0) {
    const int64_t grid = (n4 + 255) / 256;
    MOE_REQUIRE(grid < (int64_t)1 << 31, MOE_ERR_SHAPE, "moe_swiglu_backward: too many rows");
    swiglu_backward_kernel<<<(unsigned)grid, 256, 0, stream>>>(ac, dh, n4, inter, dac);
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
    const dim3 grid((total_cols + 63) / 64, (cols + 63) / 64);
    segment_transpose_kernel<<<grid, 256, 0, stream>>>(src, ld_src, src_rows, seg_offsets, dst_cols, n_segments, cols,
                                                       total_cols, dst, ld_dst, seg_stride);
  }
  return check_launch("moe_segment_transpose");
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
