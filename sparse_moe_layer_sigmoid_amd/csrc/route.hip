// moe_route: router affinities on the matrix cores, sigmoid, bias-adjusted top-K (with an
// optional group limit), normalised gates and the per-expert load histogram.
//
// "DeepSeek-V3 Technical Report" (wiki summary), "DeepSeekMoE と補助損失なしの負荷分散":
// sigmoid affinity; the bias b_i is added to the affinity only to choose the experts; the
// gates are the chosen original affinities normalised; the load is counted per batch; each
// token is limited to M = 4 nodes (here: the topk_group best of n_group expert groups).
// "FP8 混合精度訓練": the gating stays in high precision (bf16 products, fp32 sums).
//
// Design (gfx950): one workgroup of 4 waves owns TM tokens and all (<= 256) experts.  The
// TM x 256-element slice of x is staged in LDS and shared by the 4 waves; each wave owns 64
// experts and streams their router rows straight from L2 into 16x16x32 bf16 MFMAs.  The
// logits land in LDS; then each wave walks its tokens with one expert quadruple per lane
// (lane l holds experts 4l..4l+3) and picks the top-K by wave-wide argmax rounds (shuffle
// butterflies; ties to the lower index).  Loads are counted in an LDS histogram per block
// and reduced by a second one-workgroup kernel (integer sums: the result is exact and
// independent of scheduling).
#include <math.h>

#include "abi_common.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr uint32_t kNone = 0x7fffffffu;

// (v, i) beats (bv, bi): larger value, or equal value and lower index; kNone never wins.
__device__ __forceinline__ bool beats(float v, uint32_t i, float bv, uint32_t bi) {
  if (i == kNone) return false;
  if (bi == kNone) return true;
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& bv, uint32_t& bi) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const uint32_t oi = (uint32_t)__shfl_xor((int)bi, o, kWave);
    if (beats(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

template <int TM>
__global__ __launch_bounds__(256) void route_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int N, int K, int n_group, int topk_group,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    float* __restrict__ scores, int32_t* __restrict__ blk_counts) {
  constexpr int KC = 256;      // K-slice of x staged in LDS (elements)
  constexpr int XS = KC + 8;   // padded LDS row (elements): 528 B keeps MFMA reads conflict-free
  constexpr int MT = TM / 16;  // 16-token MFMA tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t xs[TM * XS];
  __shared__ float lg[TM][257];
  __shared__ int cnt[256];
  __shared__ float zg[4][256];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TM;
  cnt[tid] = 0;

  f32x4 acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15, lk = (lane >> 4) * 8;
  for (int kc0 = 0; kc0 < d; kc0 += KC) {
    const int kcn = min(KC, d - kc0);
    const int cpr = kcn / 8;
    __syncthreads();
    for (int q = tid; q < TM * cpr; q += 256) {
      const int row = q / cpr, c = q - row * cpr;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t0 + row < T) v = *(const u32x4*)(x + (size_t)(t0 + row) * d + kc0 + c * 8);
      *(u32x4*)(xs + row * XS + c * 8) = v;
    }
    __syncthreads();
    for (int kk = 0; kk < kcn; kk += 32) {
      bf16x8_t bfr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = wave * 64 + j * 16 + lrow;
        if (e < N) {
          bfr[j] = *(const bf16x8_t*)(wr + (size_t)e * d + kc0 + kk + lk);
        } else {
          bfr[j] = bf16x8_t{};
        }
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const bf16x8_t a = *(const bf16x8_t*)(xs + (i * 16 + lrow) * XS + kk + lk);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(a, bfr[j], acc[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) lg[i * 16 + (lane >> 4) * 4 + r][wave * 64 + j * 16 + lrow] = acc[i][j][r];
  __syncthreads();

  const int gs = N / n_group;
  for (int it = 0; it < TM / 4; ++it) {
    const int tl = wave + 4 * it;
    const int t = t0 + tl;
    const bool valid = t < T;  // uniform across the wave
    float s4[4], z4[4];
    bool av[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane * 4 + r;
      if (e < N) {
        const float u = lg[tl][e];
        const float s = 1.0f / (1.0f + expf(-u));
        float z = s + bias[e];
        if (z != z) z = -INFINITY;  // NaN ranks below every number
        s4[r] = s;
        z4[r] = z;
        av[r] = true;
      } else {
        s4[r] = 0.f;
        z4[r] = -INFINITY;
        av[r] = false;
      }
    }
    if (scores != nullptr && valid && lane * 4 < N)
      *(f32x4*)(scores + (size_t)t * N + lane * 4) = f32x4{s4[0], s4[1], s4[2], s4[3]};

    if (n_group > 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (lane * 4 + r < N) zg[wave][lane * 4 + r] = z4[r];
      __syncthreads();
      float gscore = -INFINITY;
      if (lane < n_group) {
        float m1 = -INFINITY, m2 = -INFINITY;
        for (int i = 0; i < gs; ++i) {
          const float v = zg[wave][lane * gs + i];
          if (v > m1) {
            m2 = m1;
            m1 = v;
          } else if (v > m2) {
            m2 = v;
          }
        }
        gscore = m1 + m2;
      }
      bool gav = lane < n_group;
      uint64_t kept = 0;
      for (int rr = 0; rr < topk_group; ++rr) {
        float bv = gscore;
        uint32_t bi = gav ? (uint32_t)lane : kNone;
        wave_argmax(bv, bi);
        if (bi == kNone) break;
        kept |= 1ull << bi;
        if ((uint32_t)lane == bi) gav = false;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (av[r] && !((kept >> ((lane * 4 + r) / gs)) & 1ull)) av[r] = false;
      __syncthreads();
    }

    float sum = 0.f;
    int my_idx[4] = {0, 0, 0, 0};
    float my_s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      float bv = 0.f;
      uint32_t bi = kNone;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (av[r] && beats(z4[r], (uint32_t)(lane * 4 + r), bv, bi)) {
          bv = z4[r];
          bi = (uint32_t)(lane * 4 + r);
        }
      wave_argmax(bv, bi);
      if (bi == kNone) break;  // cannot happen within the documented limits
      const int owner = (int)(bi >> 2), slot = (int)(bi & 3u);
      float mine = s4[0];
#pragma unroll
      for (int r = 1; r < 4; ++r)
        if (slot == r) mine = s4[r];
      const float sk = __shfl(mine, owner, kWave);
      if (lane == owner) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (slot == r) av[r] = false;
      }
      sum += sk;
      if (lane == (k & 63)) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if ((k >> 6) == q) {
            my_idx[q] = (int)bi;
            my_s[q] = sk;
          }
      }
      if (valid && lane == 0) atomicAdd(&cnt[bi], 1);
    }
    if (valid) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = q * 64 + lane;
        if (k < K) {
          topk_idx[(size_t)t * K + k] = my_idx[q];
          topk_gate[(size_t)t * K + k] = my_s[q] / sum;
        }
      }
    }
  }
  __syncthreads();
  if (tid < N) blk_counts[(size_t)blockIdx.x * N + tid] = cnt[tid];
}

__global__ __launch_bounds__(256) void counts_reduce_kernel(const int32_t* __restrict__ blk,
                                                            int nb, int N,
                                                            int32_t* __restrict__ counts) {
  const int e = threadIdx.x;
  if (e >= N) return;
  int s = 0;
  for (int b = 0; b < nb; ++b) s += blk[(size_t)b * N + e];
  counts[e] = s;
}

int route_tile(int T) { return T <= 4096 ? 16 : (T <= 8192 ? 32 : 64); }

}  // namespace
}  // namespace moe

extern "C" size_t moe_route_workspace_size(int T, int n_experts) {
  if (T < 0 || n_experts <= 0) return 0;
  const int tm = moe::route_tile(T);
  const int nb = T > 0 ? (T + tm - 1) / tm : 1;
  return (size_t)nb * (size_t)n_experts * sizeof(int32_t);
}

extern "C" moe_status moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias,
                                int T, int d, int n_experts, int top_k, int n_group,
                                int topk_group, int32_t* topk_idx, float* topk_gate,
                                int32_t* expert_counts, float* scores, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(w_router && bias && expert_counts && ws && (T == 0 || (x && topk_idx && topk_gate)),
              MOE_ERR_NULL, "moe_route: a required pointer is NULL");
  MOE_REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_route: T=%d < 0", T);
  MOE_REQUIRE(d >= 64 && d % 64 == 0, MOE_ERR_SHAPE, "moe_route: d=%d must be a positive multiple of 64", d);
  MOE_REQUIRE(n_experts >= 1 && n_experts <= 256 && n_experts % 4 == 0, MOE_ERR_SHAPE,
              "moe_route: n_experts=%d must be in [4, 256] and a multiple of 4", n_experts);
  MOE_REQUIRE(top_k >= 1 && top_k <= n_experts, MOE_ERR_SHAPE,
              "moe_route: top_k=%d must be in [1, n_experts=%d]", top_k, n_experts);
  MOE_REQUIRE(n_group >= 1 && n_group <= 64 && n_experts % n_group == 0, MOE_ERR_SHAPE,
              "moe_route: n_group=%d must divide n_experts=%d and be <= 64", n_group, n_experts);
  MOE_REQUIRE(topk_group >= 1 && topk_group <= n_group, MOE_ERR_SHAPE,
              "moe_route: topk_group=%d must be in [1, n_group=%d]", topk_group, n_group);
  if (n_group > 1) {
    MOE_REQUIRE(n_experts / n_group >= 2, MOE_ERR_SHAPE,
                "moe_route: groups need at least 2 experts (n_experts/n_group=%d)", n_experts / n_group);
    MOE_REQUIRE(top_k <= topk_group * (n_experts / n_group), MOE_ERR_SHAPE,
                "moe_route: top_k=%d exceeds the %d experts of the kept groups", top_k,
                topk_group * (n_experts / n_group));
  }
  MOE_REQUIRE(aligned16(x) && aligned16(w_router) && (scores == nullptr || aligned16(scores)),
              MOE_ERR_ALIGN, "moe_route: x, w_router and scores must be 16-byte aligned");
  const size_t need = moe_route_workspace_size(T, n_experts);
  MOE_REQUIRE(ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu bytes", ws_bytes, need);

  int32_t* blk = static_cast<int32_t*>(ws);
  const int tm = route_tile(T);
  const int nb = (T + tm - 1) / tm;
  if (nb > 0) {
    if (tm == 16)
      route_kernel<16><<<nb, 256, 0, stream>>>(x, w_router, bias, T, d, n_experts, top_k, n_group, topk_group, topk_idx, topk_gate, scores, blk);
    else if (tm == 32)
      route_kernel<32><<<nb, 256, 0, stream>>>(x, w_router, bias, T, d, n_experts, top_k, n_group, topk_group, topk_idx, topk_gate, scores, blk);
    else
      route_kernel<64><<<nb, 256, 0, stream>>>(x, w_router, bias, T, d, n_experts, top_k, n_group, topk_group, topk_idx, topk_gate, scores, blk);
  }
  counts_reduce_kernel<<<1, 256, 0, stream>>>(blk, nb, n_experts, expert_counts);
  return check_launch("moe_route");
}
