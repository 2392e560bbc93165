// moe_combine: the weighted gather back into token order, and moe_bias_update: the
// aux-loss-free load-balancing step.
//
// Combine ("DeepSeek-V3 Technical Report" (wiki summary), "DualPipe パイプライン並列化": the
// combine stage; "Vol.25 DeepSeek-V3の技術とその影響", "MoEの歴史とDeepSeekMoE-V3の特徴": the
// chosen experts return their results, merged with the always-on shared expert):
//   out[t] = y_shared[t] + sum_k gate[t,k] * y_routed[pair_pos[t,k]]   (fp32, k in order)
// An HBM-bound gather: one workgroup per token, 16-byte loads of 8 bf16 per lane, the
// token's pair rows and gates read once into LDS per workgroup, all of a thread's routed
// rows loaded before its FMAs.
//
// Bias update ("DeepSeekMoE と補助損失なしの負荷分散"): the expert's load over the batch is
// compared with the mean in integers (load * N vs T * K); an overloaded expert's bias drops
// by gamma, an underloaded one's rises by gamma, one fp32 add each.
#include "abi_common.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kMaxCombineK = 256;
constexpr int kCombineMaxThreads = 512;

// One workgroup per token: its pair rows and gates are read once into LDS; every thread owns
// 16-byte column chunks and issues the loads of all its routed rows before the FMAs (which keep
// the k order), so each thread has up to top_k gathers in flight.  The workgroup has one thread
// per two chunks of a row (d = 7168: 448 threads, each two chunks; 256 threads, which left half
// of them a fourth chunk, measured 3% slower).
template <bool OUT_F32>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const float* __restrict__ ysh,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ gate, int K,
                                                      int d, void* __restrict__ out) {
  __shared__ int s_p[kMaxCombineK];
  __shared__ float s_g[kMaxCombineK];
  const int64_t t = blockIdx.x;
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    s_p[k] = pair_pos[t * K + k];
    s_g[k] = gate[t * K + k];
  }
  __syncthreads();
  const int nc = d / 8;
  for (int c = threadIdx.x; c < nc; c += blockDim.x) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int k = k0 + q;
        const int p = k < K ? s_p[k] : -1;
        v[q] = p >= 0 ? *(const u32x4*)(y + (int64_t)p * d + c * 8) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int k = k0 + q;
        if (k < K && s_p[k] >= 0) {  // entries < 0 are skipped
          const float g = s_g[k];
          float f[8];
          unpack_bf16x8(v[q], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, f[i], acc[i]);
        }
      }
    }
    if (ysh != nullptr) {
      const f32x4 a = *(const f32x4*)(ysh + t * d + c * 8);
      const f32x4 b = *(const f32x4*)(ysh + t * d + c * 8 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += a[i];
        acc[4 + i] += b[i];
      }
    }
    if (OUT_F32) {
      float* o = static_cast<float*>(out) + t * d + c * 8;
      *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
      *(u32x4*)(static_cast<uint16_t*>(out) + t * d + c * 8) = o;
    }
  }
}

__global__ __launch_bounds__(256) void bias_update_kernel(float* __restrict__ bias,
                                                          const int32_t* __restrict__ counts,
                                                          int N, int64_t total, float gamma) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const int64_t diff = (int64_t)counts[i] * N - total;
  if (diff > 0) bias[i] = bias[i] + (-gamma);
  else if (diff < 0) bias[i] = bias[i] + gamma;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_combine(const uint16_t* y_routed, const float* y_shared,
                                  const int32_t* pair_pos, const float* topk_gate, int T,
                                  int top_k, int d, void* out, int out_dtype,
                                  hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(T == 0 || (y_routed && pair_pos && topk_gate && out), MOE_ERR_NULL,
              "moe_combine: a required pointer is NULL");
  MOE_REQUIRE(T >= 0 && top_k >= 1 && top_k <= kMaxCombineK && d >= 8 && d % 8 == 0, MOE_ERR_SHAPE,
              "moe_combine: T=%d top_k=%d d=%d (d must be a positive multiple of 8)", T, top_k, d);
  MOE_REQUIRE(out_dtype == MOE_BF16 || out_dtype == MOE_F32, MOE_ERR_DTYPE,
              "moe_combine: out_dtype must be MOE_BF16 or MOE_F32");
  MOE_REQUIRE(aligned16(y_routed) && aligned16(out) && (y_shared == nullptr || aligned16(y_shared)),
              MOE_ERR_ALIGN, "moe_combine: y_routed, y_shared and out must be 16-byte aligned");
  if (T > 0) {
    // one thread per two 8-column chunks, whole waves, 64 .. kCombineMaxThreads
    const int threads = std::min(kCombineMaxThreads, std::max(64, (d / 16 + 63) / 64 * 64));
    if (out_dtype == MOE_F32)
      combine_kernel<true><<<T, threads, 0, stream>>>(y_routed, y_shared, pair_pos, topk_gate, top_k, d, out);
    else
      combine_kernel<false><<<T, threads, 0, stream>>>(y_routed, y_shared, pair_pos, topk_gate, top_k, d, out);
  }
  return check_launch("moe_combine");
}

extern "C" moe_status moe_bias_update(float* bias, const int32_t* expert_counts, int n_experts,
                                      int64_t total_assignments, float gamma, hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(bias && expert_counts, MOE_ERR_NULL, "moe_bias_update: a required pointer is NULL");
  MOE_REQUIRE(n_experts >= 1 && n_experts <= 65536 && total_assignments >= 0, MOE_ERR_SHAPE,
              "moe_bias_update: n_experts=%d total=%lld", n_experts, (long long)total_assignments);
  MOE_REQUIRE(gamma == gamma && gamma - gamma == 0.0f, MOE_ERR_SHAPE, "moe_bias_update: gamma must be finite");
  bias_update_kernel<<<(n_experts + 255) / 256, 256, 0, stream>>>(bias, expert_counts, n_experts,
                                                                  total_assignments, gamma);
  return check_launch("moe_bias_update");
}
