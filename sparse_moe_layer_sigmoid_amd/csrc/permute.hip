// moe_permute: deterministic expert-major, token-ascending permutation of the (token, slot)
// pairs, plus the shared expert's identity segment -- the within-GPU half of the dispatch
// stage in "DeepSeek-V3 Technical Report" (wiki summary), "DualPipe パイプライン並列化";
// every pair gets a row ("DeepSeekMoE と補助損失なしの負荷分散": no token is dropped).
//
// Design: blocks of 256 tokens, one token per lane.  For each expert a block keeps one
// 64-bit lane mask per wave (ds_or_b64 into LDS); the rank of a pair among the block's pairs
// of the same expert is popcount(masks of earlier waves) + popcount(own mask below the
// lane), so the order never depends on atomic timing.  Three kernels: per-block counts,
// a one-workgroup scan (over blocks per expert, then over experts), and the scatter.
#include "abi_common.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kTok = 256;  // tokens per block

__device__ __forceinline__ void build_masks(unsigned long long (*masks)[256],
                                            const int32_t* __restrict__ idx, int T, int K,
                                            int N, int t, int wave, int lane) {
  for (int e = threadIdx.x; e < 4 * 256; e += kTok) (&masks[0][0])[e] = 0ull;
  __syncthreads();
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = idx[(size_t)t * K + k];
      if (e >= 0 && e < N) atomicOr(&masks[wave][e], 1ull << lane);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTok) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                             int T, int K, int N,
                                                             int32_t* __restrict__ blk_cnt) {
  __shared__ unsigned long long masks[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kTok + threadIdx.x;
  build_masks(masks, idx, T, K, N, t, wave, lane);
  for (int e = threadIdx.x; e < N; e += kTok)
    blk_cnt[(size_t)blockIdx.x * N + e] = __popcll(masks[0][e]) + __popcll(masks[1][e]) +
                                          __popcll(masks[2][e]) + __popcll(masks[3][e]);
}

// One workgroup: blk_base[b][e] = sum_{b' < b} blk_cnt[b'][e] (the scatter adds offsets[e]),
// offsets = exclusive scan of the expert totals.  The block counts are read 16 at a time, so
// the loads of a thread are in flight together rather than one per loop trip.
__global__ __launch_bounds__(256) void permute_scan_kernel(const int32_t* __restrict__ blk_cnt,
                                                           int32_t* __restrict__ blk_base,
                                                           int nb, int N, int T, int n_shared,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int tot[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < N) {
    constexpr int kBatch = 16;
    for (int b0 = 0; b0 < nb; b0 += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) c[i] = b0 + i < nb ? blk_cnt[(size_t)(b0 + i) * N + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (b0 + i < nb) blk_base[(size_t)(b0 + i) * N + e] = run;
        run += c[i];
      }
    }
  }
  tot[e] = (e < N) ? run : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over the 256 expert totals
  for (int o = 1; o < 256; o <<= 1) {
    const int v = (e >= o) ? tot[e - o] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  const int excl = tot[e] - ((e < N) ? run : 0);
  if (e < N) offsets[e] = excl;
  if (e == 0) {
    const int routed = tot[255];
    offsets[N] = routed;
    if (n_shared) offsets[N + 1] = routed + T;
  }
}

__global__ __launch_bounds__(kTok) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int T, int K, int N, int n_shared,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ pair_pos) {
  __shared__ unsigned long long masks[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kTok + threadIdx.x;
  build_masks(masks, idx, T, K, N, t, wave, lane);
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int k = 0; k < K; ++k) {
    const int e = idx[(size_t)t * K + k];
    int pos = -1;
    if (e >= 0 && e < N) {
      pos = offsets[e] + blk_base[(size_t)blockIdx.x * N + e];
      for (int w = 0; w < wave; ++w) pos += __popcll(masks[w][e]);
      pos += __popcll(masks[wave][e] & below);
      sorted_token[pos] = t;
    }
    pair_pos[(size_t)t * K + k] = pos;
  }
  if (n_shared) sorted_token[(size_t)offsets[N] + t] = t;
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_permute_workspace_size(int T, int n_experts) {
  if (T < 0 || n_experts <= 0) return 0;
  const int nb = T > 0 ? (T + moe::kTok - 1) / moe::kTok : 1;
  return 2 * (size_t)nb * (size_t)n_experts * sizeof(int32_t);
}

extern "C" moe_status moe_permute(const int32_t* topk_idx, int T, int top_k, int n_experts,
                                  int n_shared, int32_t* expert_offsets, int32_t* sorted_token,
                                  int32_t* pair_pos, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(expert_offsets && ws && (T == 0 || (topk_idx && sorted_token && pair_pos)), MOE_ERR_NULL,
              "moe_permute: a required pointer is NULL");
  MOE_REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_permute: T=%d < 0", T);
  MOE_REQUIRE(n_experts >= 1 && n_experts <= 256, MOE_ERR_SHAPE,
              "moe_permute: n_experts=%d must be in [1, 256]", n_experts);
  MOE_REQUIRE(top_k >= 1 && top_k <= n_experts, MOE_ERR_SHAPE,
              "moe_permute: top_k=%d must be in [1, n_experts=%d]", top_k, n_experts);
  MOE_REQUIRE(n_shared == 0 || n_shared == 1, MOE_ERR_SHAPE, "moe_permute: n_shared=%d must be 0 or 1", n_shared);
  MOE_REQUIRE((int64_t)T * (top_k + n_shared) < (int64_t)1 << 31, MOE_ERR_SHAPE,
              "moe_permute: T*(top_k+n_shared) overflows 32-bit row indices");
  const size_t need = moe_permute_workspace_size(T, n_experts);
  MOE_REQUIRE(ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_permute: workspace %zu < %zu bytes", ws_bytes, need);

  const int nb = (T + kTok - 1) / kTok;
  int32_t* blk_cnt = static_cast<int32_t*>(ws);
  int32_t* blk_base = blk_cnt + (size_t)(nb > 0 ? nb : 1) * n_experts;
  if (nb > 0) permute_count_kernel<<<nb, kTok, 0, stream>>>(topk_idx, T, top_k, n_experts, blk_cnt);
  permute_scan_kernel<<<1, 256, 0, stream>>>(blk_cnt, blk_base, nb, n_experts, T, n_shared, expert_offsets);
  if (nb > 0)
    permute_scatter_kernel<<<nb, kTok, 0, stream>>>(topk_idx, T, top_k, n_experts, n_shared, blk_base,
                                                    expert_offsets, sorted_token, pair_pos);
  return check_launch("moe_permute");
}
