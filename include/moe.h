/*
 * moe.h -- C ABI of libmoe.so: the forward pass of one DeepSeekMoE layer on one MI355X
 * (gfx950), with sigmoid routing, the aux-loss-free routing bias and its load-driven
 * update, in bf16 and in FP8 (E4M3) with 1x128 / 128x128 scaling.
 *
 * Sources: "DeepSeek-V3 Technical Report" (wiki summary page), sections
 * "DeepSeekMoE と補助損失なしの負荷分散" and "FP8 混合精度訓練"; "Vol.25 DeepSeek-V3の技術と
 * その影響", section "MoEの歴史とDeepSeekMoE-V3の特徴".
 *
 * Conventions shared by every entry point
 *  - Every call returns a moe_status.  Arguments are checked on the host, synchronously,
 *    before anything is launched; on an error nothing is launched and nothing is written,
 *    and moe_last_error() (thread-local) describes the problem.
 *  - Work is enqueued asynchronously on the caller's HIP stream; no call synchronises the
 *    device or reads device memory back to the host.  A fault inside a kernel surfaces at
 *    the caller's next synchronisation.
 *  - Ownership: every pointer is caller-owned memory; pointers documented as "device" must
 *    be device memory of the current device.  The library never allocates or frees device
 *    memory and keeps no state between calls.  Scratch memory comes from the caller's
 *    workspace, sized by the *_workspace_size() queries; for moe_route and moe_permute it need
 *    not be initialised and its contents are undefined after the call; moe_grouped_gemm's
 *    small workspace holds counters that must be zero when a call starts and that every call
 *    leaves at zero (see there).  Calls that may run at the same time (on streams not ordered
 *    with each other) need distinct workspaces; calls on one stream may share one.
 *  - Layout: row-major and contiguous unless an ld* (leading dimension, in elements) is
 *    given.  Device pointers must be 16-byte aligned; leading dimensions must keep every
 *    row 16-byte aligned.
 *  - Types: bf16 tensors are passed as uint16_t (the bfloat16 bit pattern); FP8 tensors as
 *    uint8_t holding OCP E4M3FN codes (bias 7, largest finite 448, no infinities, 0x7F /
 *    0xFF NaN); scales are float32.
 *  - Rows of the expert GEMMs follow the permutation of moe_permute: pairs sorted by expert
 *    then token ("sorted rows"), followed by one segment of all T tokens for the shared
 *    expert, whose group index is n_experts.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* a size is out of range or inconsistent */
  MOE_ERR_DTYPE = 3,     /* unsupported dtype / epilogue combination */
  MOE_ERR_ALIGN = 4,     /* a pointer or leading dimension breaks 16-byte alignment */
  MOE_ERR_WORKSPACE = 5, /* workspace missing or smaller than the query returned */
  MOE_ERR_HIP = 6        /* a HIP launch reported an error */
};

enum { MOE_BF16 = 0, MOE_F32 = 1, MOE_FP8_E4M3 = 2 };
enum { MOE_EPI_NONE = 0, MOE_EPI_SWIGLU = 1 };
/* Scale formats of FP8 tensors: float32 scales, or E8M0 codes (uint8, value 2^(code-127)). */
enum { MOE_SCALE_F32 = 0, MOE_SCALE_E8M0 = 1 };

/* Human-readable name of a status code (static string). */
const char* moe_status_str(moe_status s);
/* Detail of the last error returned on this thread ("" if none). */
const char* moe_last_error(void);
/* Version of this ABI (bumped on any incompatible change). */
int moe_abi_version(void);

/* ------------------------------------------------------------------------------------
 * moe_route -- router affinities, bias-adjusted top-K selection, gates, expert loads.
 * "DeepSeek-V3 Technical Report", "DeepSeekMoE と補助損失なしの負荷分散": the token-to-
 * expert affinity is a sigmoid, s[t,i] = sigmoid(x_t . e_i); the per-expert bias b_i is
 * added to the affinity only to decide the routing, z = s + b; the gates are the selected
 * ORIGINAL affinities normalised to sum to one; the load of every expert is counted over
 * the whole batch.  With n_group > 1 the selection is first limited to the topk_group
 * groups (of n_experts/n_group contiguous experts) with the largest sum of their two best
 * z -- the single-GPU stand-in for the node limit M = 4 of the same section.
 * Precision ("FP8 混合精度訓練": gating stays in high precision): the affinities come from
 * bf16 products with fp32 sums promoted out of the matrix cores every 256 elements; sigmoid,
 * z, the selection and the gates are fp32.  A token whose fp32 decision margin (gap between
 * the K-th and (K+1)-th z, or half the gap between the last kept and best dropped group
 * score) is below 4e-6 is recomputed entirely in fp64 (exact products, fp64 sums, sigmoid,
 * selection and gates), so the chosen experts match an fp64 evaluation of the definition.
 * Equal z: the lower expert index wins (likewise for equal group scores).
 *
 *   x           device bf16 [T, d]
 *   w_router    device bf16 [n_experts, d] (row i = e_i)
 *   bias        device f32 [n_experts]
 *   topk_idx    device i32 [T, top_k] out: selected experts, descending z
 *   topk_gate   device f32 [T, top_k] out: gates (sum to 1 per token)
 *   expert_counts device i32 [n_experts] out: load per expert (overwritten)
 *   scores      device f32 [T, n_experts] out, optional (NULL): the affinities s
 *   ws          device workspace of moe_route_workspace_size(T, n_experts) bytes
 * Limits: 0 <= T; 64 <= d, d % 64 == 0; 4 <= n_experts <= 256, n_experts % 4 == 0;
 * 1 <= top_k <= n_experts; n_group in 1..64 dividing n_experts, with n_experts/n_group a
 * power of two >= 4 when n_group > 1; 1 <= topk_group <= n_group;
 * top_k <= topk_group*n_experts/n_group; ws 16-byte aligned.
 * T == 0 writes zero counts only; x, topk_idx and topk_gate may then be NULL.
 * ------------------------------------------------------------------------------------ */
size_t moe_route_workspace_size(int T, int n_experts);
moe_status moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T,
                     int d, int n_experts, int top_k, int n_group, int topk_group,
                     int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                     float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_route_noalloc -- moe_route for callers that cannot allocate device memory: code
 * running under HIP graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and checks as moe_route without the workspace: its
 * scratch is a static device array of the library, one copy per device (8.4 MB, held until
 * the process ends), whose device address is looked up once per device on the first call
 * there.  The call allocates nothing.
 * Limits: those of moe_route, and T <= MOE_ROUTE_NOALLOC_MAX_T (1024 tokens); a larger T
 * returns MOE_ERR_SHAPE with nothing launched.  Every call initialises the scratch it reads,
 * but all calls on one device share that array: calls that may overlap in time on one
 * device (unordered streams) race and must not be issued. */
#define MOE_ROUTE_NOALLOC_MAX_T 1024
moe_status moe_route_noalloc(const uint16_t* x, const uint16_t* w_router, const float* bias, int T,
                             int d, int n_experts, int top_k, int n_group, int topk_group,
                             int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                             float* scores, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_permute -- token permutation for the expert GEMMs (the within-GPU half of the
 * dispatch stage of "DeepSeek-V3 Technical Report", "DualPipe パイプライン並列化").
 * Pairs (t, k) are ordered by expert, then by token (deterministic, no atomics order),
 * followed (n_shared == 1) by a segment holding every token once, in order, for the
 * shared expert.  No token is dropped ("トークンドロップなし"): there is no capacity limit.
 * The loads are recomputed here from topk_idx.
 *
 *   topk_idx        device i32 [T, top_k]; every token's entries must be distinct experts
 *                   in [0, n_experts) (as moe_route produces).  An entry outside that range
 *                   is skipped: its pair_pos is -1 and it takes no row.
 *   expert_offsets  device i32 [n_experts + n_shared + 1] out: group g's rows are
 *                   [off[g], off[g+1]); the shared expert is group n_experts.
 *   sorted_token    device i32 [T * (top_k + n_shared)] out: token of each sorted row.
 *   pair_pos        device i32 [T, top_k] out: sorted row of pair (t, k).
 * Limits: 0 <= T; 1 <= top_k <= n_experts <= 256; n_shared in {0, 1}.  With T == 0 only the
 * offsets are written (all zero) and topk_idx, sorted_token and pair_pos may be NULL.
 * ------------------------------------------------------------------------------------ */
size_t moe_permute_workspace_size(int T, int n_experts);
moe_status moe_permute(const int32_t* topk_idx, int T, int top_k, int n_experts, int n_shared,
                       int32_t* expert_offsets, int32_t* sorted_token, int32_t* pair_pos,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * fp8_quant_1x128 -- online quantisation of activations in 1x128 tiles.
 * "DeepSeek-V3 Technical Report", "FP8 混合精度訓練": activations are scaled per 1x128
 * tile ("細粒度量子化") from the tile's current max |x| ("オンライン量子化") and stored
 * as E4M3 ("E4M3 統一").  For each tile: s = fl32(amax / 448) (IEEE division; an
 * all-zero tile gets s = 1) and q = RNE_E4M3(fl32(x / s)), saturating at +/-448; the code's
 * sign bit is x's sign bit.
 *
 *   x      device bf16 [rows, cols], leading dimension ldx (elements, >= cols)
 *   q      device u8 [rows, cols] out (contiguous)
 *   scale  device f32 [rows, cols/128] out
 * Limits: rows >= 0; cols >= 128, cols % 128 == 0; ldx % 8 == 0.
 * ------------------------------------------------------------------------------------ */
moe_status fp8_quant_1x128(const uint16_t* x, int rows, int cols, int64_t ldx, uint8_t* q,
                           float* scale, hipStream_t stream);

/* fp8_quant_128x128 -- the weight counterpart (one-time weight preparation, not on the
 * per-batch path): n_mats matrices [n, k], one scale per 128x128 block, same rounding.
 *   w      device bf16 [n_mats, n, k];  q device u8 [n_mats, n, k] out;
 *   scale  device f32 [n_mats, n/128, k/128] out.
 * Limits: n_mats >= 0; n, k >= 128 and multiples of 128. */
moe_status fp8_quant_128x128(const uint16_t* w, int n_mats, int n, int k, uint8_t* q,
                             float* scale, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * fp8_quant_1x128_e8m0 / fp8_quant_128x128_e8m0 -- the same tiles with a power-of-two
 * scale ("Vol.25 DeepSeek-V3の技術とその影響", "学習と推論の課題と解決策": the values of a
 * 1x128 / 128x128 tile can share one exponent; "DeepSeek-V3 Technical Report", "考察", and
 * the talk's "ハードウェアデザインへの提案": tile / block scaling supported by the matrix
 * unit itself).  For each tile: k = the smallest integer with amax <= 448 * 2^k, clamped
 * to [-127, 127] (k = 0 for an all-zero tile); scale code = k + 127 (E8M0, value
 * 2^(code-127)); q = RNE_E4M3(x * 2^-k) (an exact product), the code's sign bit being x's.
 * Arguments and limits as fp8_quant_1x128 / fp8_quant_128x128, with the scales written as
 * uint8 codes: [rows, cols/128] and [n_mats, n/128, k/128].
 * ------------------------------------------------------------------------------------ */
moe_status fp8_quant_1x128_e8m0(const uint16_t* x, int rows, int cols, int64_t ldx, uint8_t* q,
                                uint8_t* scale, hipStream_t stream);

/* fp8_dequant_1x128 -- the inverse view: out = RNE_bf16(decode(q) * scale) per 1x128 tile (the
 * FP8 backward's Wgrad takes the stored E4M3 h of the forward this way).
 *   q device u8 [rows, cols]; scale device f32 [rows, cols/128]; out device bf16 [rows, cols].
 * Limits: rows >= 0; cols >= 128, cols % 128 == 0. */
moe_status fp8_dequant_1x128(const uint8_t* q, const float* scale, int rows, int cols,
                             uint16_t* out, hipStream_t stream);
moe_status fp8_quant_128x128_e8m0(const uint16_t* w, int n_mats, int n, int k, uint8_t* q,
                                  uint8_t* scale, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_grouped_gemm -- one GEMM per expert over that expert's sorted rows:
 *   out[r, :] = A[r, :] . W[g]^T   for every row r of group g,
 * the expert FFN layers of "DeepSeek-V3 Technical Report", "DeepSeekMoE と補助損失なしの
 * 負荷分散" (expert width 2048).  With epilogue SWIGLU the GEMM is the gate/up projection:
 * W[g] holds W1 in rows [0, N/2) and W3 in rows [N/2, N), and the stored output is
 * h = silu(A W1^T) * (A W3^T), N/2 columns wide.  On the FP8 path ("FP8 混合精度訓練")
 * A and W are E4M3 with one scale per 1x128 tile of A and per 128x128 block of W; every
 * 128-element slice of K is multiplied on the matrix cores and its partial sum is scaled
 * by s_A * s_W and added to an fp32 accumulator (the N_C = 128 promotion interval).  An
 * FP8 output (the gate/up projection feeding the down projection) is quantised per 1x128
 * tile exactly as fp8_quant_1x128 does.  bf16 inputs accumulate in fp32.
 * With scale_fmt = MOE_SCALE_E8M0 every FP8 scale (a_scale, w_scale, out_scale) is an E8M0
 * code (uint8, same shapes) as fp8_quant_*_e8m0 writes them: the matrix cores apply the
 * power-of-two scales of both operands to each 128-element slice and accumulate straight
 * into fp32 (no separate promotion step), and an FP8 output is quantised as
 * fp8_quant_1x128_e8m0 does.
 *
 * Rows: group g (first_group <= g < first_group + n_groups) owns the sorted rows
 * [group_offsets[g], group_offsets[g+1]).  Row r reads A row a_rows[r] when a_rows is not
 * NULL (gather, e.g. a_rows = sorted_token and A = x), else A row r (A holds every sorted
 * row, e.g. h); it writes out row r - group_offsets[first_group].  Groups are read on
 * the device; empty groups cost nothing.  m_total must equal group_offsets[first_group +
 * n_groups] - group_offsets[first_group] (it sizes the launch; the device values decide
 * the work).
 * ------------------------------------------------------------------------------------ */
typedef struct moe_gemm_desc {
  int in_dtype;                 /* MOE_BF16 or MOE_FP8_E4M3 (both A and W) */
  const void* a;                /* device A [*, K], leading dimension lda (elements) */
  const void* a_scale;          /* FP8: device [*, K/128] scales (row-aligned with A), f32 or
                                   E8M0 per scale_fmt; else NULL */
  const int32_t* a_rows;        /* device i32 gather index per sorted row, or NULL */
  int64_t lda;
  const void* w;                /* device W [G][N][K] contiguous, G > last group used */
  const void* w_scale;          /* FP8: device [G][N/128][K/128] scales per scale_fmt; else NULL */
  const int32_t* group_offsets; /* device i32, at least first_group + n_groups + 1 entries */
  int first_group;
  int n_groups;                 /* 1..1024 */
  int64_t m_total;              /* rows covered by the groups (see above) */
  int N;                        /* rows of each W[g] (2*I for SWIGLU) */
  int K;                        /* reduction length */
  int epilogue;                 /* MOE_EPI_NONE or MOE_EPI_SWIGLU */
  void* out;                    /* device output, leading dimension ldo (elements) */
  int out_dtype;                /* MOE_BF16, MOE_F32, or MOE_FP8_E4M3 (+ out_scale) */
  int64_t ldo;
  void* out_scale;              /* FP8 output: device [rows, out_cols/128] scales per scale_fmt */
  /* Optional split output: the last tail_groups groups write f32 rows to out_tail (row r of
   * such a group lands in out_tail row r - group_offsets[first_group + n_groups - tail_groups],
   * leading dimension ldo_tail) instead of out; the other groups write out as above.  One
   * launch then covers the routed experts (bf16 rows) and the shared expert (f32 rows).
   * tail_groups = 0 disables it (out_tail ignored). */
  int tail_groups;
  void* out_tail;
  int64_t ldo_tail;
  int scale_fmt;                /* MOE_SCALE_F32 (0) or MOE_SCALE_E8M0 (FP8 only) */
  int64_t ldw;                  /* row stride of each W[g] in elements (0: K); W[g] starts at
                                   w + g * N * ldw */
  void* ws;                     /* device workspace of moe_grouped_gemm_workspace_size() bytes,
                                   16-byte aligned, zero-filled before its first use */
  size_t ws_bytes;
  /* Optional ragged reduction (f32 output, epilogue NONE, f32 scales), for weight gradients
   * whose reduction axis is each expert's own rows ("FP8 混合精度訓練": Wgrad): device i32,
   * at least first_group + n_groups + 1 non-decreasing entries, or NULL.  Group g then sums only
   * over K columns [0, k_g), k_g = len_g = k_offsets[g+1] - k_offsets[g] rounded up to the K
   * step (64 bf16 / 128 FP8 elements), at least one step and at most K; columns [len_g, k_g) of
   * A and W must hold zeros (the segment transposes write them) for the exact sum over len_g.
   * Columns at and beyond k_g are not read. */
  const int32_t* k_offsets;
  /* Optional with SWIGLU: device f32 [rows, ldo_preact] out, or NULL: the gate and up products
   * themselves (a = A W1^T in columns [0, N/2), c = A W3^T in [N/2, N), the fp32 values the
   * epilogue takes, bit for bit those of the same launch without SwiGLU and with an f32
   * output), for a training forward whose backward needs them (the SwiGLU backward takes a and
   * c; "DeepSeek-V3 Technical Report", "FP8 混合精度訓練": activations cached for the backward).
   * Row r lands in row r - group_offsets[first_group].  16-byte aligned, ldo_preact >= N and a
   * multiple of 4. */
  void* out_preact;
  int64_t ldo_preact;
} moe_gemm_desc;
/* Limits: K a positive multiple of 64 (bf16) or 128 (FP8); N a positive multiple of 128 (bf16)
 * or 256 (FP8) -- with SWIGLU that is N/2 a multiple of 64 or 128; FP8 input needs a_scale and
 * w_scale (4-byte aligned); an FP8 output needs FP8 input, SWIGLU and out_scale; SWIGLU
 * output is bf16 or FP8; 1 <= n_groups <= 1024; 0 <= m_total < 2^31; one W[g] < 2 GiB;
 * lda/ldo keep rows 16-byte aligned.  A split output (tail_groups > 0) needs epilogue NONE,
 * out_dtype MOE_BF16, tail_groups <= n_groups and a 16-byte aligned out_tail with
 * ldo_tail >= N.  E8M0 scales need K a multiple of 512 (each scale row is read 4 codes at a
 * time). */
/* Workspace of moe_grouped_gemm (256 bytes): arrival counters with which the workgroups of a
 * launch keep in step, so that the rows of one expert that several workgroups process meet its
 * weights in the same L2 (used by the bf16 SwiGLU launches with 128-row blocks).  The caller
 * zero-fills it once; every call leaves it zero-filled again.  Calls that may overlap in time
 * need distinct workspaces (sharing one could only make the bounded waits run to their bound,
 * never change a result); calls on one stream may share one.  Missing or too small ->
 * MOE_ERR_WORKSPACE. */
size_t moe_grouped_gemm_workspace_size(void);
moe_status moe_grouped_gemm(const moe_gemm_desc* desc, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_combine -- the weighted sum back into token order (the combine stage of
 * "DeepSeek-V3 Technical Report", "DualPipe パイプライン並列化"; "Vol.25", "MoEの歴史と
 * DeepSeekMoE-V3の特徴": the chosen experts' results are merged with the shared expert):
 *   out[t] = y_shared[t] + sum_k gate[t,k] * y_routed[pair_pos[t,k]]
 * accumulated in fp32 in the order k = 0..top_k-1 (acc = fma(gate, y, acc)), then the
 * shared term added; stored as bf16 (round to nearest even) or f32.
 *   y_routed  device bf16 [T*top_k (sorted rows), d]
 *   y_shared  device f32 [T, d] or NULL (no shared expert)
 *   pair_pos  device i32 [T, top_k] (entries < 0 are skipped)
 *   topk_gate device f32 [T, top_k]
 *   out       device [T, d], bf16 or f32 per out_dtype
 * Limits: T >= 0; 1 <= top_k <= 256; d >= 8, d % 8 == 0.
 * ------------------------------------------------------------------------------------ */
moe_status moe_combine(const uint16_t* y_routed, const float* y_shared, const int32_t* pair_pos,
                       const float* topk_gate, int T, int top_k, int d, void* out,
                       int out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * moe_bias_update -- the aux-loss-free load-balancing step ("DeepSeek-V3 Technical
 * Report", "DeepSeekMoE と補助損失なしの負荷分散": monitor each expert's load over the
 * batch; lower an overloaded expert's bias by gamma, raise an underloaded one's):
 *   b_i <- b_i - gamma * sign(load_i - total/N)
 * decided in integers (load_i * N vs total_assignments), one fp32 add of -gamma or +gamma;
 * an expert exactly at the mean keeps its bias bit for bit.
 *   bias           device f32 [n_experts], updated in place
 *   expert_counts  device i32 [n_experts] (the loads, e.g. from moe_route)
 *   total_assignments  T * top_k
 * Limits: 1 <= n_experts <= 65536; total_assignments >= 0; gamma finite.
 * ------------------------------------------------------------------------------------ */
moe_status moe_bias_update(float* bias, const int32_t* expert_counts, int n_experts,
                           int64_t total_assignments, float gamma, hipStream_t stream);

/* ====================================================================================
 * Backward pass.  "DeepSeek-V3 Technical Report", "FP8 混合精度訓練": a training step runs
 * the layer's Fprop, Dgrad and Wgrad GEMMs.  The gradients are the chain rule of the forward
 * definition ("DeepSeekMoE と補助損失なしの負荷分散"): with L = sum(d_out * out), gates
 * g_k = s_k / S over the selected affinities (S = their sum) and the selection (and bias)
 * carrying no gradient:
 *   dy = g * d_out at a routed pair's sorted row, d_out at the token's shared row;
 *   dg_k = <d_out, y_k>;  du_k = s_k (1 - s_k) (dg_k - sum_j g_j dg_j) / S;
 *   per expert: dh = dy W2, [da | dc] = [dh c silu'(a) | dh silu(a)], dx_rows = [da | dc] W13,
 *   dW2 = dy^T h, dW13 = [da | dc]^T x_rows;  router: dx += sum_k du_k e_{idx_k},
 *   dW_r[idx_k] += du_k x.
 * The GEMMs run on moe_grouped_gemm (Dgrad with transposed weights, Wgrad per expert over
 * transposed row segments, see moe_segment_transpose); the calls below are the pieces
 * between them.
 * ==================================================================================== */

/* moe_combine_backward -- the combine's and router's gradients for every token t.  A pair the
 * permutation skipped (pair_pos < 0) contributes nothing: its du is 0 and no dy row is written.
 *   d_out     device bf16 [T, d]: gradient of the layer output
 *   y_routed  device bf16 [T*top_k, d]: the forward's routed expert outputs (sorted rows)
 *   topk_idx, topk_gate, pair_pos: the forward's routing and permutation ([T, top_k])
 *   scores    device f32 [T, n_experts]: the forward's affinities s (moe_route's scores)
 *   dy        device bf16 [T*(top_k+1), d] out: rows pair_pos[t,k] = RNE(g_k d_out[t]), rows
 *             T*top_k + t = d_out[t] (the down projection's input gradient, sorted rows)
 *   du        device f32 [T, top_k] out: router logit gradients of the selected experts
 *   du_row    device f32 [T*top_k] out: du by sorted row (du_row[pair_pos[t,k]] = du[t,k])
 *   dy_q, dy_scale  NULL, or device u8 [T*(top_k+1), d] and f32 [T*(top_k+1), d/128] out: the
 *             written dy rows also as E4M3 with 1x128 scales, the codes fp8_quant_1x128 gives on
 *             them (the FP8 path's Dgrad operand, "FP8 混合精度訓練")
 * dg is accumulated in fp32 in a fixed order; the rest is fp32.  Limits: T >= 0;
 * 1 <= top_k <= min(32, n_experts); d >= 8, d % 8 == 0 (d % 128 == 0 with dy_q); routing and
 * permutation as moe_route and moe_permute produce them (valid, distinct experts).  With T == 0
 * nothing is done. */
moe_status moe_combine_backward(const uint16_t* d_out, const uint16_t* y_routed,
                                const int32_t* topk_idx, const float* topk_gate,
                                const float* scores, const int32_t* pair_pos, int T, int top_k,
                                int d, int n_experts, uint16_t* dy, float* du, float* du_row,
                                uint8_t* dy_q, float* dy_scale, hipStream_t stream);

/* moe_swiglu_backward -- through h = silu(a) c, elementwise over rows x inter:
 *   da = dh c sig(a) (1 + a (1 - sig(a))),  dc = dh a sig(a)   (fp32, stored RNE bf16)
 *   ac   device f32 [rows, 2*inter]: a in columns [0, inter), c in [inter, 2*inter)
 *        (the gate/up GEMM without its SwiGLU epilogue)
 *   dh   device f32 [rows, inter]
 *   dac  device bf16 [rows, 2*inter] out: da | dc
 *   dac_q, dac_scale  NULL, or device u8 [rows, 2*inter] and f32 [rows, 2*inter/128] out: dac
 *        also as E4M3 with 1x128 scales, the codes fp8_quant_1x128 gives on it
 * Limits: rows >= 0; inter >= 4, inter % 4 == 0 (inter % 128 == 0 with dac_q). */
moe_status moe_swiglu_backward(const float* ac, const float* dh, int64_t rows, int inter,
                               uint16_t* dac, uint8_t* dac_q, float* dac_scale, hipStream_t stream);

/* moe_segment_transpose -- row segments of a bf16 matrix become zero-padded column blocks of
 * its transpose: for segment g (rows [seg_offsets[g], seg_offsets[g+1]) of the logical
 * source), column dst_cols[g] + i of dst holds source row seg_offsets[g] + i (read through
 * src_rows if not NULL) for i < the segment's length, and zeros up to dst_cols[g+1].
 * With seg_stride > 0 each segment instead gets its own block: element (c, i) of segment g
 * at dst + g * seg_stride + c * ld_dst + i, i < dst_cols[g+1] - dst_cols[g] (equal widths make
 * [n_segments][cols][width] operands for one grouped GEMM over all segments).
 *   src         device bf16, rows of `cols` elements, leading dimension ld_src
 *   src_rows    device i32 gather index per logical row, or NULL
 *   seg_offsets device i32 [n_segments+1];  dst_cols device i32 [n_segments+1], non-decreasing,
 *               dst_cols[g+1] - dst_cols[g] >= the segment's length, dst_cols[n_segments] =
 *               total_cols
 *   dst         device bf16 [cols, ld_dst] out (columns [0, total_cols) written)
 * Limits: n_segments >= 1; cols and total_cols multiples of 8; with seg_stride > 0 the
 * dst_cols entries are multiples of 8; leading dimensions keep rows 16-byte aligned.  (Used for
 * the bf16 Wgrad operands and, once, for transposed weight copies.) */
moe_status moe_segment_transpose(const uint16_t* src, int64_t ld_src, const int32_t* src_rows,
                                 const int32_t* seg_offsets, const int32_t* dst_cols,
                                 int n_segments, int cols, int total_cols, uint16_t* dst,
                                 int64_t ld_dst, int64_t seg_stride, hipStream_t stream);

/* moe_segment_transpose_fp8 -- the Wgrad operands of the FP8 path ("FP8 混合精度訓練": Wgrad in
 * E4M3 on transposed operands; "考察" asks for the transposition and the quantisation to be
 * fused): segment g's rows become block g of q, [n_segments][cols][width] E4M3 codes, element
 * (c, i) = source row seg_offsets[g] + i (through src_rows if not NULL), channel c, for i below
 * the segment's length and zero beyond, quantised as fp8_quant_1x128 / fp8_quant_128x128 would
 * quantise that bf16 block matrix (the same scales and codes, bit for bit):
 *   block_scales = 0: 1x128 along the width; scale [n_segments * cols][width / 128] (the A
 *                     operand of a Wgrad GEMM, the [n_segments * cols, width] view);
 *   block_scales = 1: 128x128 blocks; scale [n_segments][cols / 128][width / 128] (its B operand).
 *   src         device bf16, rows of `cols` elements, leading dimension ld_src
 *   src_rows    device i32 gather index per logical row, or NULL
 *   seg_offsets device i32 [n_segments + 1], non-decreasing; each segment at most `width` rows
 *   q           device u8 [n_segments][cols][width] out;  scale device f32 out (above)
 * Limits: n_segments >= 1; cols and width positive multiples of 128; ld_src >= cols, a multiple
 * of 8; src 16-byte, q 8-byte, scale 4-byte aligned. */
moe_status moe_segment_transpose_fp8(const uint16_t* src, int64_t ld_src, const int32_t* src_rows,
                                     const int32_t* seg_offsets, int n_segments, int cols, int width,
                                     int block_scales, uint8_t* q, float* scale, hipStream_t stream);

/* moe_router_wgrad -- dW_r[e] = sum over expert e's sorted rows r of du_row[r] x[sorted_token[r]]
 * (fp32, rows in order).
 *   x device bf16 [T, d]; sorted_token, expert_offsets from moe_permute; du_row from
 *   moe_combine_backward; dw_router device f32 [n_experts, d] out (overwritten).
 * Limits: 1 <= n_experts <= 65535; d % 8 == 0. */
moe_status moe_router_wgrad(const uint16_t* x, const int32_t* sorted_token,
                            const int32_t* expert_offsets, const float* du_row, int n_experts,
                            int d, float* dw_router, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
