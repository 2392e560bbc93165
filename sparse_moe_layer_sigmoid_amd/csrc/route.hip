// moe_route: router affinities, sigmoid, bias-adjusted top-K (with an optional group
// limit), normalised gates and the per-expert load histogram.
//
// "DeepSeek-V3 Technical Report" (wiki summary), "DeepSeekMoE と補助損失なしの負荷分散":
// sigmoid affinity; the bias b_i is added to the affinity only to choose the experts; the
// gates are the chosen original affinities normalised; the load is counted per batch; each
// token is limited to M = 4 nodes (here: the topk_group best of n_group expert groups).
// "FP8 混合精度訓練": the gating stays in high precision (bf16 products, fp32 or better sums,
// partial sums promoted out of the matrix cores every 256 elements).
//
// Five kernels:
//  1. logits: a split-K MFMA GEMM.  A workgroup (8 waves of 64 tokens x 64 experts) owns 128
//     tokens x all experts x one K slice; x and router rows are staged through LDS in 128-byte
//     K steps (double buffered, XOR-swizzled, global loads issued two steps ahead); every 256
//     elements of K the 16x16x32 bf16 MFMA partial sum is added into an fp32 accumulator (the
//     matrix cores truncate inside their adder, so long chains are avoided).  Partial logits of
//     each slice go to the workspace.
//  2. select: one wave per token (lane l holds experts 4l..4l+3) sums the slices in a fixed
//     order, forms s and z, picks the top-K by wave-wide argmax rounds (ties to the lower
//     index) and measures the decision margin: the gap between the K-th and (K+1)-th z, and
//     between the last kept and the best dropped group score.
//  3. refine: tokens whose fp32 margin is below kRefineGap (listed by the select kernel) are
//     recomputed in fp64 (exact bf16 products, fp64 sums, fp64 sigmoid and selection), so the
//     choice of experts does not depend on the matrix cores' rounding: their fp64 logits by
//     workgroups of (listed token, 16 experts) into the workspace (the split-K partials are
//     dead by then), then one wave per listed token selects.
//  4. count: each block of 64 tokens histograms its tokens' experts.
//  5. reduce: one wave per expert sums the block histograms (integer sums: exact).
#include <math.h>

#include <mutex>

#include "abi_common.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr uint32_t kNone = 0x7fffffffu;
constexpr float kRefineGap = 4e-6f;  // fp32 decision margin below which a token is redone in fp64
constexpr int kTM = 128;             // tokens per logits workgroup (the router rows are re-read once per kTM tokens)
constexpr int kRows = kTM + 256;     // LDS rows per stage: kTM tokens + 256 router rows
constexpr int kLogitsThreads = 512;  // 8 waves: 2 token halves x 4 expert quarters, 64 x 64 each
constexpr int kChunks = kRows * 8 / kLogitsThreads;  // 16-byte chunks per thread per stage

template <typename V>
__device__ __forceinline__ bool beats(V v, uint32_t i, V bv, uint32_t bi) {
  if (i == kNone) return false;
  if (bi == kNone) return true;
  return v > bv || (v == bv && i < bi);
}

template <typename V>
__device__ __forceinline__ void wave_argmax(V& bv, uint32_t& bi) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const V ov = __shfl_xor(bv, o, kWave);
    const uint32_t oi = (uint32_t)__shfl_xor((int)bi, o, kWave);
    if (beats(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

template <typename V>
__device__ __forceinline__ V sigmoid_v(V u);
template <>
__device__ __forceinline__ float sigmoid_v<float>(float u) { return 1.0f / (1.0f + expf(-u)); }
template <>
__device__ __forceinline__ double sigmoid_v<double>(double u) { return 1.0 / (1.0 + exp(-u)); }

// Selection for one token by one wave.  u[r] is the logit of expert 4*lane + r.  Writes the
// outputs when `write`; returns the decision margin (min of the expert gap and half the
// group gap), +inf when nothing competes.
template <typename V>
__device__ V select_token(const V u[4], const float* __restrict__ bias, int N, int K, int n_group,
                          int topk_group, int64_t t, bool write, int32_t* __restrict__ topk_idx,
                          float* __restrict__ topk_gate, float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const V inf = (V)INFINITY;
  V s4[4], z4[4];
  bool av[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = lane * 4 + r;
    if (e < N) {
      const V s = sigmoid_v<V>(u[r]);
      V z = s + (V)bias[e];
      if (z != z) z = -inf;  // NaN ranks below every number
      s4[r] = s;
      z4[r] = z;
      av[r] = true;
    } else {
      s4[r] = (V)0;
      z4[r] = -inf;
      av[r] = false;
    }
  }
  if (write && scores != nullptr && lane * 4 < N)
    *(f32x4*)(scores + t * N + lane * 4) = f32x4{(float)s4[0], (float)s4[1], (float)s4[2], (float)s4[3]};

  V margin = inf;
  if (n_group > 1) {
    const int gs = N / n_group;  // a power of two >= 4: a lane's four experts share a group
    const int lanes_per_group = gs >> 2;
    const int g = (lane * 4) / gs;
    V m1 = -inf, m2 = -inf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const V v = z4[r];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    for (int o = 1; o < lanes_per_group; o <<= 1) {
      const V p1 = __shfl_xor(m1, o, kWave), p2 = __shfl_xor(m2, o, kWave);
      const V lo = m1 < p1 ? m1 : p1;
      const V hi2 = m2 > p2 ? m2 : p2;
      m1 = m1 > p1 ? m1 : p1;
      m2 = lo > hi2 ? lo : hi2;
    }
    const bool leader = (lane % lanes_per_group) == 0 && g < n_group;
    const V gscore = m1 + m2;
    bool gav = leader;
    uint64_t kept = 0;
    V last = (V)0;
    for (int rr = 0; rr <= topk_group; ++rr) {
      if (rr == n_group) break;
      V bv = gscore;
      uint32_t bi = gav ? (uint32_t)g : kNone;
      wave_argmax(bv, bi);
      if (bi == kNone) break;
      if (rr == topk_group) {
        margin = (last - bv) * (V)0.5;  // a group score moves twice as much as one z
        break;
      }
      kept |= 1ull << bi;
      last = bv;
      if (gav && (uint32_t)g == bi) gav = false;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (av[r] && !((kept >> g) & 1ull)) av[r] = false;
  }

  V sum = (V)0, zk = (V)0;
  int my_idx[4] = {0, 0, 0, 0};
  V my_s[4] = {(V)0, (V)0, (V)0, (V)0};
  for (int k = 0; k <= K; ++k) {
    V bv = (V)0;
    uint32_t bi = kNone;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (av[r] && beats(z4[r], (uint32_t)(lane * 4 + r), bv, bi)) {
        bv = z4[r];
        bi = (uint32_t)(lane * 4 + r);
      }
    wave_argmax(bv, bi);
    if (bi == kNone) break;
    if (k == K) {  // the best expert left out: the decision margin
      const V gap = zk - bv;
      margin = gap < margin ? gap : margin;
      break;
    }
    zk = bv;
    const int owner = (int)(bi >> 2), slot = (int)(bi & 3u);
    V mine = s4[0];
#pragma unroll
    for (int r = 1; r < 4; ++r)
      if (slot == r) mine = s4[r];
    const V sk = __shfl(mine, owner, kWave);
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
  }
  if (write) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = q * 64 + lane;
      if (k < K) {
        topk_idx[t * K + k] = my_idx[q];
        topk_gate[t * K + k] = (float)(my_s[q] / sum);
      }
    }
  }
  return margin;
}

// ---- kernel 1: split-K logits ----
__global__ __launch_bounds__(kLogitsThreads) void route_logits_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           int T, int d, int N, int splits,
                                                           float* __restrict__ part,
                                                           int32_t* __restrict__ n_flagged) {
  constexpr int STAGE = kRows * 128;
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_flagged = 0;  // the select kernel appends after this one
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // token half, expert quarter
  const int tile = blockIdx.x / splits, split = blockIdx.x - tile * splits;
  const int t0 = tile * kTM;
  const int nsteps_all = d / 64;
  const int ks0 = (int)((int64_t)split * nsteps_all / splits);
  const int ks1 = (int)((int64_t)(split + 1) * nsteps_all / splits);
  const int cch = tid & 7;
  // kChunks chunks of 16 B per thread per stage: rows r = tid/8 + 64 i: [0, kTM) tokens, then router
  const uint8_t* src[kChunks];
  bool live[kChunks];
  int dst[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int r = (tid >> 3) + (kLogitsThreads / 8) * i;
    if (r < kTM) {
      live[i] = t0 + r < T;
      src[i] = reinterpret_cast<const uint8_t*>(x + (int64_t)min(t0 + r, T - 1) * d) + cch * 16;
    } else {
      const int e = r - kTM;
      live[i] = e < N;
      src[i] = reinterpret_cast<const uint8_t*>(wr + (int64_t)min(e, N - 1) * d) + cch * 16;
    }
    dst[i] = r * 128 + ((cch ^ (r & 7)) << 4);
  }
  // two register sets: the global loads of step ks + 2 are issued while step ks computes and
  // step ks + 1's data, loaded a step earlier, moves to LDS, so each load has two steps to land
  u32x4 rA[kChunks], rB[kChunks];
  // (the loads are unconditional -- rows past T or N read a clamped valid row -- and the dead
  // rows are zeroed as they go to LDS, so no branch hides the loads' counts from the waits)
  auto gload = [&](u32x4 (&reg)[kChunks], int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) reg[i] = *(const u32x4*)(src[i] + (int64_t)ks * 128);
  };
  auto sstore = [&](const u32x4 (&reg)[kChunks], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      *(u32x4*)(smem + buf * STAGE + dst[i]) = live[i] ? reg[i] : u32x4{0u, 0u, 0u, 0u};
  };
  f32x4 acc[4][4], prt[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = prt[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lr = lane & 15, lg = lane >> 4;
  // (every step issues its loads, the last steps re-reading step ks1 - 1, so the number of
  // loads in flight is the same on every path and the waits can leave the newer ones pending)
  if (ks0 < ks1) {
    gload(rA, ks0);
    sstore(rA, 0);
    gload(rB, min(ks0 + 1, ks1 - 1));
  }
  __syncthreads();
  // step ks: LDS buffer (ks - ks0) & 1 holds its data, `nxt` holds step ks + 1's, `fre` is free
  auto step = [&](int ks, u32x4 (&nxt)[kChunks], u32x4 (&fre)[kChunks]) __attribute__((always_inline)) {
    const int cur = (ks - ks0) & 1;
    gload(fre, min(ks + 2, ks1 - 1));
    const uint8_t* S = smem + cur * STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = h * 4 + lg;
      bf16x8_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + lr;
        af[i] = *(const bf16x8_t*)(S + r * 128 + ((ch ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = kTM + wn * 64 + j * 16 + lr;
        bf[j] = *(const bf16x8_t*)(S + r * 128 + ((ch ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) prt[i][j] = mfma_bf16(af[i], bf[j], prt[i][j]);
    }
    const bool more = ks + 1 < ks1;
    if (((ks + 1) & 3) == 0 || !more) {  // promote every 256 elements of K
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += prt[i][j];
          prt[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (more) sstore(nxt, cur ^ 1);
    __syncthreads();
  };
  int ks = ks0;
  for (; ks + 1 < ks1; ks += 2) {
    step(ks, rB, rA);
    step(ks + 1, rA, rB);
  }
  if (ks < ks1) step(ks, rB, rA);
  float* out = part + (int64_t)split * T * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + wm * 64 + i * 16 + lg * 4 + r;
      if (t < T) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[(int64_t)t * 256 + wn * 64 + j * 16 + lr] = acc[i][j][r];
      }
    }
}

// ---- kernel 2: fp32 selection, one wave per token ----
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ part, int splits,
                                                           const float* __restrict__ bias, int T, int N,
                                                           int K, int n_group, int topk_group,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_gate,
                                                           float* __restrict__ scores,
                                                           int32_t* __restrict__ n_flagged,
                                                           int32_t* __restrict__ flagged) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves leave together
  const int lane = threadIdx.x & 63;
  float u[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const f32x4 v = *(const f32x4*)(part + ((int64_t)s * T + t) * 256 + lane * 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] += v[r];
  }
  const float margin = select_token<float>(u, bias, N, K, n_group, topk_group, t, true, topk_idx, topk_gate, scores);
  if (lane == 0 && margin < kRefineGap) flagged[atomicAdd(n_flagged, 1)] = (int32_t)t;
}

// ---- kernel 3a: fp64 logits of the flagged (near-tie) tokens ----
// Workgroup (x, y) takes listed tokens x, x + gridDim.x, ... and experts 16y .. 16y + 15: wave
// w computes experts 16y + w + 4j (j < 4) side by side; its lanes split K into 16-byte chunks
// (lane l takes chunks l, l + 64, ...) and keep eight independent fp64 partial sums per expert
// (one per element of a chunk), so the fp64 adds pipeline, and each pass loads kRefineU chunks
// of the token and of the four expert rows before using any, so that the pass waits for one
// memory latency rather than one per chunk and expert.  Spreading a token over N / 16
// workgroups keeps the router-row reads (the whole W_r per token) off one CU.  Each logit
// depends on its token and expert alone, so the list's order does not matter.
constexpr int kRefineChunk = 16;  // experts per workgroup
constexpr int kRefineU = 3;       // chunks per lane per pass
__global__ __launch_bounds__(256) void route_refine_logits_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr, int d, int N,
                                                                  const int32_t* __restrict__ n_flagged,
                                                                  const int32_t* __restrict__ flagged,
                                                                  double* __restrict__ l64) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nf = *n_flagged;
  const int nd = d / 8;  // 16-byte chunks per row
  const uint16_t* er[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) er[j] = wr + (int64_t)min(blockIdx.y * kRefineChunk + wave + 4 * j, N - 1) * d;
  for (int i = blockIdx.x; i < nf; i += gridDim.x) {
    const int64_t t = flagged[i];
    const uint16_t* xr = x + t * d;
    double a[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 8; ++q) a[j][q] = 0.0;
    for (int c0 = lane; c0 < nd; c0 += 64 * kRefineU) {
      u32x4 xv[kRefineU], ev[kRefineU][4];
#pragma unroll
      for (int u = 0; u < kRefineU; ++u) {  // chunks past the row re-read its last one, unused
        const int c = min(c0 + 64 * u, nd - 1);
        xv[u] = *(const u32x4*)(xr + c * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) ev[u][j] = *(const u32x4*)(er[j] + c * 8);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the pass's loads together, ahead of their uses
#pragma unroll
      for (int u = 0; u < kRefineU; ++u) {
        // a chunk past the row adds +0 (no branch, so the loads above stay batched; the sums
        // start at +0 and never become -0, so adding +0 leaves them unchanged)
        if (c0 + 64 * u >= nd) xv[u] = u32x4{0u, 0u, 0u, 0u};
        float xf[8];
        unpack_bf16x8(xv[u], xf);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float ef[8];
          unpack_bf16x8(ev[u][j], ef);
#pragma unroll
          for (int q = 0; q < 8; ++q) a[j][q] += (double)(xf[q] * ef[q]);  // bf16 products are exact in fp32
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      double sum = ((a[j][0] + a[j][1]) + (a[j][2] + a[j][3])) + ((a[j][4] + a[j][5]) + (a[j][6] + a[j][7]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
      const int e = blockIdx.y * kRefineChunk + wave + 4 * j;
      if (lane == 0 && e < N) l64[(int64_t)i * 256 + e] = sum;
    }
  }
}

// ---- kernel 3b: fp64 selection and gates of the flagged tokens, one wave per token ----
__global__ __launch_bounds__(256) void route_refine_select_kernel(const float* __restrict__ bias, int N, int K,
                                                                  int n_group, int topk_group,
                                                                  const int32_t* __restrict__ n_flagged,
                                                                  const int32_t* __restrict__ flagged,
                                                                  const double* __restrict__ l64,
                                                                  int32_t* __restrict__ topk_idx,
                                                                  float* __restrict__ topk_gate,
                                                                  float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int nf = *n_flagged;
  for (int i = blockIdx.x * 4 + (threadIdx.x >> 6); i < nf; i += gridDim.x * 4) {
    const int64_t t = flagged[i];
    double u[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] = (lane * 4 + r < N) ? l64[(int64_t)i * 256 + lane * 4 + r] : 0.0;
    select_token<double>(u, bias, N, K, n_group, topk_group, t, true, topk_idx, topk_gate, scores);
  }
}

// ---- kernel 4: per-block load histogram (64 tokens per block) ----
__global__ __launch_bounds__(64) void route_count_kernel(const int32_t* __restrict__ topk_idx, int T, int N, int K,
                                                         int32_t* __restrict__ blk_counts) {
  __shared__ int cnt[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < N; e += 64) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  if (t < T)
    for (int k = 0; k < K; ++k) atomicAdd(&cnt[topk_idx[t * K + k]], 1);
  __syncthreads();
  for (int e = lane; e < N; e += 64) blk_counts[(int64_t)blockIdx.x * N + e] = cnt[e];
}

// ---- kernel 5: one wave per expert sums the block histograms ----
__global__ __launch_bounds__(64) void counts_reduce_kernel(const int32_t* __restrict__ blk, int nb, int N,
                                                           int32_t* __restrict__ counts) {
  const int e = blockIdx.x, lane = threadIdx.x;
  int s = 0;
  for (int b = lane; b < nb; b += 64) s += blk[(int64_t)b * N + e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (lane == 0) counts[e] = s;
}

constexpr int route_splits(int T, int d) {
  const int tiles = (T + kTM - 1) / kTM;
  int s = tiles > 0 ? 512 / tiles : 1;
  // up to 8 K slices per 128-token tile; decode-sized batches (one or two tiles) take up to 16,
  // so that they still spread over 16-32 workgroups (T = 256: 36.8 -> 34.0 us per call; 32
  // slices make the selection's sum of the slices cost more than the logits save)
  const int cap = tiles <= 2 ? 16 : 8;
  s = s < 1 ? 1 : (s > cap ? cap : s);
  return s > d / 64 ? d / 64 : s;
}

struct RouteWs {
  size_t part_off, nflag_off, list_off, blk_off, total;
};

constexpr RouteWs route_ws(int T, int d, int N) {
  RouteWs w{};
  const int S = route_splits(T, d);
  const int nb = T > 0 ? (T + 63) / 64 : 1;
  w.part_off = 0;  // split-K partials, then the fp64 logits of the flagged tokens
  w.nflag_off = (size_t)(S > 2 ? S : 2) * (size_t)T * 256 * sizeof(float);
  w.list_off = w.nflag_off + 256;
  w.blk_off = w.list_off + (((size_t)T * sizeof(int32_t) + 255) & ~(size_t)255);
  w.total = w.blk_off + (size_t)nb * (size_t)N * sizeof(int32_t);
  return w;
}

// Scratch of moe_route_noalloc: the workspace of moe_route for up to kNoAllocMaxT tokens and
// 256 experts, as a static device array (one per device, held until the process ends: 8.4 MB).
// Host code reaches it only through the address hipGetSymbolAddress gives for the current
// device; the array's name is not a device address on the host.
constexpr int kNoAllocMaxT = MOE_ROUTE_NOALLOC_MAX_T;
constexpr size_t kNoAllocBytes = route_ws(kNoAllocMaxT, 1 << 20, 256).total;
__device__ __align__(256) uint8_t scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
moe_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  MOE_REQUIRE(e == hipSuccess, MOE_ERR_HIP, "moe_route_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_HIP, "moe_route_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    MOE_REQUIRE(e == hipSuccess && ptr != nullptr, MOE_ERR_HIP, "moe_route_noalloc: hipGetSymbolAddress: %s",
                hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

moe_status route_check(const char* fn, const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int d,
                       int n_experts, int top_k, int n_group, int topk_group, const int32_t* topk_idx,
                       const float* topk_gate, const int32_t* expert_counts, const float* scores) {
  MOE_REQUIRE(w_router && bias && expert_counts && (T == 0 || (x && topk_idx && topk_gate)),
              MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  MOE_REQUIRE(T >= 0, MOE_ERR_SHAPE, "%s: T=%d < 0", fn, T);
  MOE_REQUIRE(d >= 64 && d % 64 == 0, MOE_ERR_SHAPE, "%s: d=%d must be a positive multiple of 64", fn, d);
  MOE_REQUIRE(n_experts >= 4 && n_experts <= 256 && n_experts % 4 == 0, MOE_ERR_SHAPE,
              "%s: n_experts=%d must be in [4, 256] and a multiple of 4", fn, n_experts);
  MOE_REQUIRE(top_k >= 1 && top_k <= n_experts, MOE_ERR_SHAPE,
              "%s: top_k=%d must be in [1, n_experts=%d]", fn, top_k, n_experts);
  MOE_REQUIRE(n_group >= 1 && n_group <= 64 && n_experts % n_group == 0, MOE_ERR_SHAPE,
              "%s: n_group=%d must divide n_experts=%d and be <= 64", fn, n_group, n_experts);
  MOE_REQUIRE(topk_group >= 1 && topk_group <= n_group, MOE_ERR_SHAPE,
              "%s: topk_group=%d must be in [1, n_group=%d]", fn, topk_group, n_group);
  if (n_group > 1) {
    const int gs = n_experts / n_group;
    MOE_REQUIRE(gs >= 4 && (gs & (gs - 1)) == 0, MOE_ERR_SHAPE,
                "%s: groups must hold a power of two >= 4 experts (n_experts/n_group=%d)", fn, gs);
    MOE_REQUIRE(top_k <= topk_group * gs, MOE_ERR_SHAPE,
                "%s: top_k=%d exceeds the %d experts of the kept groups", fn, top_k, topk_group * gs);
  }
  MOE_REQUIRE(aligned16(x) && aligned16(w_router) && (scores == nullptr || aligned16(scores)),
              MOE_ERR_ALIGN, "%s: x, w_router and scores must be 16-byte aligned", fn);
  return MOE_OK;
}

// The five kernels of one routing call, their scratch laid out in `ws` (route_ws bytes).
void route_launch(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int d, int n_experts,
                  int top_k, int n_group, int topk_group, int32_t* topk_idx, float* topk_gate,
                  int32_t* expert_counts, float* scores, void* ws, hipStream_t stream) {
  const RouteWs L = route_ws(T, d, n_experts);
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* part = reinterpret_cast<float*>(base + L.part_off);
  int32_t* n_flagged = reinterpret_cast<int32_t*>(base + L.nflag_off);
  int32_t* flagged = reinterpret_cast<int32_t*>(base + L.list_off);
  int32_t* blk = reinterpret_cast<int32_t*>(base + L.blk_off);
  const int S = route_splits(T, d);
  const int tiles = (T + kTM - 1) / kTM;
  const int nb = (T + 63) / 64;
  if (T > 0) {
    route_logits_kernel<<<tiles * S, kLogitsThreads, 0, stream>>>(x, w_router, T, d, n_experts, S, part, n_flagged);
    route_select_kernel<<<(T + 3) / 4, 256, 0, stream>>>(part, S, bias, T, n_experts, top_k, n_group, topk_group,
                                                         topk_idx, topk_gate, scores, n_flagged, flagged);
    double* l64 = reinterpret_cast<double*>(part);  // the partials are consumed by now
    route_refine_logits_kernel<<<dim3(T < 64 ? T : 64, (n_experts + kRefineChunk - 1) / kRefineChunk), 256, 0, stream>>>(
        x, w_router, d, n_experts, n_flagged, flagged, l64);
    route_refine_select_kernel<<<(T + 3) / 4 < 256 ? (T + 3) / 4 : 256, 256, 0, stream>>>(
        bias, n_experts, top_k, n_group, topk_group, n_flagged, flagged, l64, topk_idx, topk_gate, scores);
    route_count_kernel<<<nb, 64, 0, stream>>>(topk_idx, T, n_experts, top_k, blk);
  }
  counts_reduce_kernel<<<n_experts, 64, 0, stream>>>(blk, nb, n_experts, expert_counts);
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_route_workspace_size(int T, int n_experts) {
  if (T < 0 || n_experts <= 0) return 0;
  // sized for the largest split count (d only limits it further)
  return moe::route_ws(T, 1 << 20, n_experts).total;
}

extern "C" moe_status moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias,
                                int T, int d, int n_experts, int top_k, int n_group,
                                int topk_group, int32_t* topk_idx, float* topk_gate,
                                int32_t* expert_counts, float* scores, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  using namespace moe;
  clear_error();
  const moe_status st = route_check("moe_route", x, w_router, bias, T, d, n_experts, top_k, n_group, topk_group,
                                    topk_idx, topk_gate, expert_counts, scores);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(ws, MOE_ERR_NULL, "moe_route: a required pointer is NULL");
  const size_t need = moe_route_workspace_size(T, n_experts);
  MOE_REQUIRE(ws_bytes >= need && aligned16(ws), MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu bytes (or unaligned)",
              ws_bytes, need);
  route_launch(x, w_router, bias, T, d, n_experts, top_k, n_group, topk_group, topk_idx, topk_gate, expert_counts,
               scores, ws, stream);
  return check_launch("moe_route");
}

extern "C" moe_status moe_route_noalloc(const uint16_t* x, const uint16_t* w_router, const float* bias,
                                        int T, int d, int n_experts, int top_k, int n_group,
                                        int topk_group, int32_t* topk_idx, float* topk_gate,
                                        int32_t* expert_counts, float* scores, hipStream_t stream) {
  using namespace moe;
  clear_error();
  const moe_status st = route_check("moe_route_noalloc", x, w_router, bias, T, d, n_experts, top_k, n_group,
                                    topk_group, topk_idx, topk_gate, expert_counts, scores);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(T <= kNoAllocMaxT, MOE_ERR_SHAPE, "moe_route_noalloc: T=%d exceeds the static scratch (T <= %d)", T,
              kNoAllocMaxT);
  static_assert(route_ws(kNoAllocMaxT, 1 << 20, 256).total == kNoAllocBytes, "scratch sized for the largest call");
  MOE_REQUIRE(route_ws(T, d, n_experts).total <= kNoAllocBytes, MOE_ERR_SHAPE,
              "moe_route_noalloc: T=%d needs more scratch than the static array holds", T);
  void* ws = nullptr;
  const moe_status se = scratch_of_current_device(&ws);
  if (se != MOE_OK) return se;
  route_launch(x, w_router, bias, T, d, n_experts, top_k, n_group, topk_group, topk_idx, topk_gate, expert_counts,
               scores, ws, stream);
  return check_launch("moe_route_noalloc");
}
