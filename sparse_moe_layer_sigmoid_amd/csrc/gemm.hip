// moe_grouped_gemm: one GEMM per expert over its sorted rows, on the gfx950 matrix cores.
//
// What it computes ("DeepSeek-V3 Technical Report" (wiki summary)):
//  * "DeepSeekMoE と補助損失なしの負荷分散" -- every expert is a feed-forward block of width
//    2048; the gate/up projection is fused with the SwiGLU product h = silu(a W1^T)*(a W3^T).
//  * "FP8 混合精度訓練" -- E4M3 operands with one scale per 1x128 activation tile and per
//    128x128 weight block ("細粒度量子化"); every 128-element slice of K is one
//    16x16x128 MFMA whose partial sum is scaled by s_A * s_W and added to an fp32
//    accumulator ("高精度累積", N_C = 128); the gate/up output feeding the down projection
//    is re-quantised per 1x128 tile in the epilogue ("オンライン量子化").
//
// Design (CDNA4 first):
//  * A workgroup owns a BM x BN output tile of one expert.  Tiles are found on the device:
//    each workgroup scans the group offsets (one wave, shuffles) to map its linear index to
//    (expert, row block); the launch is sized by an upper bound, surplus workgroups exit.
//  * Each K step moves 128 bytes per row (64 bf16 or 128 E4M3) of A and W through LDS with
//    16-byte loads, double buffered (prefetch into registers during the MFMAs, one barrier
//    per step).  LDS rows are 128 B with the 16-byte chunks XOR-swizzled by (row & 7) so the
//    MFMA operand reads (16 rows x one chunk) hit distinct banks.
//  * A rows are gathered through the permutation (token -> sorted row) while loading; rows
//    past the end of an expert's segment re-read a valid row and are not stored.
//  * SwiGLU: the B tile holds BN/2 gate rows then the matching BN/2 up rows, and each wave
//    owns matching gate and up columns, so h is formed in registers.
//  * Outputs are staged through LDS and written as full 16-byte row chunks (bf16 and fp8);
//    fp32 outputs are written straight from the accumulators.
#include <math.h>

#include "abi_common.h"
#include "device_common.h"

namespace moe {
namespace {

enum { OUT_BF16 = 0, OUT_F32 = 1, OUT_FP8 = 2 };

struct GemmArgs {
  const uint8_t* a;
  const float* a_scale;
  const int32_t* a_rows;
  int64_t lda_b;      // bytes per A row
  const uint8_t* w;
  const float* w_scale;
  const int32_t* offs;  // group_offsets + first_group (n_groups + 1 entries)
  int first_group;
  int n_groups;
  int N;              // rows of each W[g]
  int ksteps;         // number of 128-byte K steps
  int ksb;            // K / 128: scale columns (FP8)
  int64_t w_row_b;    // bytes per W row
  int n_tiles;        // output tiles along N
  uint8_t* out;
  int64_t ldo_b;      // bytes per output row
  float* out_scale;
  int out_scale_ld;
};

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

template <int BM, int BN, int WGM, int WGN, bool FP8, bool SWIGLU, int OUT>
__global__ __launch_bounds__(WGM * WGN * 64) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM;  // rows per wave
  constexpr int WN = BN / WGN;  // W rows (output columns; gate+up for SwiGLU) per wave
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_CPT = BM * 8 / NT, B_CPT = BN * 8 / NT;
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  constexpr int OC = SWIGLU ? BN / 2 : BN;  // output columns of a tile
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile / thread mismatch");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(!SWIGLU || TN % 2 == 0, "SwiGLU waves need matching gate and up tiles");
  static_assert(OUT != OUT_FP8 || (FP8 && SWIGLU && OC == 128), "fp8 output = one 1x128 tile per row");
  static_assert(!FP8 || (SWIGLU ? WN / 2 <= 128 : WN <= 128), "a wave must sit inside one 128-row scale block");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ float s_as[FP8 ? 2 * BM : 1];
  __shared__ float s_red[OUT == OUT_FP8 ? WGN * BM : 1];
  __shared__ int s_info[3];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave - wm * WGN;
  const int mt = blockIdx.x / p.n_tiles;
  const int nt = blockIdx.x - mt * p.n_tiles;

  // ---- map this workgroup's row block to (group, first row, valid rows) ----
  if (wave == 0) {
    const int G = p.n_groups;
    const int per = (G + 63) >> 6;
    const int g0 = min(G, lane * per), g1 = min(G, g0 + per);
    int local = 0;
    for (int g = g0; g < g1; ++g) local += (p.offs[g + 1] - p.offs[g] + BM - 1) / BM;
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, 63, kWave);
    if (lane == 0 && mt >= total) s_info[0] = -1;
    int run = incl - local;
    if (mt >= run && mt < incl) {
      for (int g = g0; g < g1; ++g) {
        const int c = (p.offs[g + 1] - p.offs[g] + BM - 1) / BM;
        if (mt < run + c) {
          const int r0 = p.offs[g] + (mt - run) * BM;
          s_info[0] = g;
          s_info[1] = r0;
          s_info[2] = min(BM, p.offs[g + 1] - r0);
          break;
        }
        run += c;
      }
    }
  }
  __syncthreads();
  const int gl = s_info[0];
  if (gl < 0) return;
  const int row0 = s_info[1], nrows = s_info[2];
  const int g = p.first_group + gl;
  const int base_row = p.offs[0];

  // ---- per-thread global sources and LDS destinations ----
  const int cch = tid & 7;
  const uint8_t* a_src[A_CPT];
  int a_lds[A_CPT];
#pragma unroll
  for (int i = 0; i < A_CPT; ++i) {
    const int rr = (tid >> 3) + i * (NT / 8);
    const int r = row0 + min(rr, nrows - 1);
    const int64_t src = p.a_rows ? (int64_t)p.a_rows[r] : (int64_t)r;
    a_src[i] = p.a + src * p.lda_b + cch * 16;
    a_lds[i] = rr * 128 + ((cch ^ (rr & 7)) << 4);
  }
  const uint8_t* wg = p.w + (int64_t)g * p.N * p.w_row_b;
  const uint8_t* b_src[B_CPT];
  int b_lds[B_CPT];
#pragma unroll
  for (int i = 0; i < B_CPT; ++i) {
    const int rr = (tid >> 3) + i * (NT / 8);
    int n;
    if (SWIGLU) n = (rr < BN / 2) ? nt * (BN / 2) + rr : p.N / 2 + nt * (BN / 2) + (rr - BN / 2);
    else n = nt * BN + rr;
    b_src[i] = wg + (int64_t)n * p.w_row_b + cch * 16;
    b_lds[i] = A_BYTES + rr * 128 + ((cch ^ (rr & 7)) << 4);
  }
  const float* sa_src = nullptr;
  const float* sw_a = nullptr;  // scale row of this wave's (gate) columns
  const float* sw_b = nullptr;  // scale row of this wave's up columns (SwiGLU)
  if (FP8) {
    if (tid < BM) {
      const int r = row0 + min(tid, nrows - 1);
      const int64_t src = p.a_rows ? (int64_t)p.a_rows[r] : (int64_t)r;
      sa_src = p.a_scale + src * p.ksb;
    }
    const float* swg = p.w_scale + (int64_t)g * (p.N / 128) * p.ksb;
    if (SWIGLU) {
      sw_a = swg + (int64_t)((nt * (BN / 2) + wn * (WN / 2)) / 128) * p.ksb;
      sw_b = swg + (int64_t)((p.N / 2 + nt * (BN / 2) + wn * (WN / 2)) / 128) * p.ksb;
    } else {
      sw_a = swg + (int64_t)((nt * BN + wn * WN) / 128) * p.ksb;
      sw_b = sw_a;
    }
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[A_CPT], rb[B_CPT];
  float rsa = 0.f;
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_CPT; ++i) ra[i] = *(const u32x4*)(a_src[i] + (int64_t)kt * 128);
#pragma unroll
    for (int i = 0; i < B_CPT; ++i) rb[i] = *(const u32x4*)(b_src[i] + (int64_t)kt * 128);
    if (FP8 && tid < BM) rsa = sa_src[kt];
  };
  auto sstore = [&](int buf) {
    uint8_t* s = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_CPT; ++i) *(u32x4*)(s + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_CPT; ++i) *(u32x4*)(s + b_lds[i]) = rb[i];
    if (FP8 && tid < BM) s_as[buf * BM + tid] = rsa;
  };

  const int lr = lane & 15, lg = lane >> 4;
  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = wm * WM + i * 16 + lr;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if (SWIGLU) b_row[j] = (j < TN / 2) ? wn * (WN / 2) + j * 16 + lr : BN / 2 + wn * (WN / 2) + (j - TN / 2) * 16 + lr;
    else b_row[j] = wn * WN + j * 16 + lr;
  }

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < p.ksteps; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < p.ksteps;
    if (more) gload(kt + 1);
    const uint8_t* As = smem + cur * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    if (!FP8) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ch = ks * 4 + lg;
        bf16x8_t af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = *(const bf16x8_t*)(As + a_row[i] * 128 + ((ch ^ (a_row[i] & 7)) << 4));
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[j] = *(const bf16x8_t*)(Bs + b_row[j] * 128 + ((ch ^ (b_row[j] & 7)) << 4));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma_bf16(af[i], bfr[j], acc[i][j]);
      }
    } else {
      const int ch = lg * 2;
      i32x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint8_t* rowp = As + a_row[i] * 128;
        const u32x4 lo = *(const u32x4*)(rowp + ((ch ^ (a_row[i] & 7)) << 4));
        const u32x4 hi = *(const u32x4*)(rowp + (((ch + 1) ^ (a_row[i] & 7)) << 4));
        af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint8_t* rowp = Bs + b_row[j] * 128;
        const u32x4 lo = *(const u32x4*)(rowp + ((ch ^ (b_row[j] & 7)) << 4));
        const u32x4 hi = *(const u32x4*)(rowp + (((ch + 1) ^ (b_row[j] & 7)) << 4));
        bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      const float swa = sw_a[kt], swb = sw_b[kt];
      const float* sas = s_as + cur * BM;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float sa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sa[r] = sas[wm * WM + i * 16 + lg * 4 + r];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float sw = (SWIGLU && j >= TN / 2) ? swb : swa;
          const f32x4 part = mfma_fp8(af[i], bfr[j], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(part[r], sa[r] * sw, acc[i][j][r]);
        }
      }
    }
    if (more) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  constexpr int TO = SWIGLU ? TN / 2 : TN;  // output 16-column tiles per wave
  const int64_t orow0 = (int64_t)(row0 - base_row);
  float v[TM][TO][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TO; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        v[i][j][r] = SWIGLU ? silu(acc[i][j][r]) * acc[i][j + TO][r] : acc[i][j][r];
  const int col_w = SWIGLU ? wn * (WN / 2) : wn * WN;  // first output column of this wave

  if (OUT == OUT_F32) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = wm * WM + i * 16 + lg * 4 + r;
        if (m < nrows) {
          float* o = reinterpret_cast<float*>(p.out + (orow0 + m) * p.ldo_b) + nt * OC + col_w + lr;
#pragma unroll
          for (int j = 0; j < TO; ++j) o[j * 16] = v[i][j][r];
        }
      }
    return;
  }

  constexpr int ESZ = (OUT == OUT_BF16) ? 2 : 1;
  constexpr int SROW = OC * ESZ + 16;  // staged row pitch (bytes)
  static_assert(BM * SROW <= 2 * STAGE, "staging does not fit");
  uint8_t* stage = smem;
  if (OUT == OUT_BF16) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = wm * WM + i * 16 + lg * 4 + r;
#pragma unroll
        for (int j = 0; j < TO; ++j)
          *reinterpret_cast<uint16_t*>(stage + m * SROW + (col_w + j * 16 + lr) * 2) = (uint16_t)f32_to_bf16_rne(v[i][j][r]);
      }
  } else {  // OUT_FP8: per-row amax over the tile's 128 columns, then E4M3 codes
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < TO; ++j) mx = fmaxf(mx, fabsf(v[i][j][r]));
        mx = max16(mx);
        if (lr == 0) s_red[wn * BM + wm * WM + i * 16 + lg * 4 + r] = mx;
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = wm * WM + i * 16 + lg * 4 + r;
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < WGN; ++q) amax = fmaxf(amax, s_red[q * BM + m]);
        const float s = (amax == 0.f) ? 1.0f : amax / 448.0f;
#pragma unroll
        for (int j = 0; j < TO; ++j) stage[m * SROW + col_w + j * 16 + lr] = (uint8_t)f32_to_e4m3(v[i][j][r] / s);
        if (wn == 0 && lr == 0 && m < nrows) p.out_scale[(orow0 + m) * p.out_scale_ld + nt] = s;
      }
  }
  __syncthreads();
  constexpr int CPR = OC * ESZ / 16;  // 16-byte chunks per output row
  for (int q = tid; q < nrows * CPR; q += NT) {
    const int m = q / CPR, c = q - m * CPR;
    *(u32x4*)(p.out + (orow0 + m) * p.ldo_b + (int64_t)nt * OC * ESZ + c * 16) = *(const u32x4*)(stage + m * SROW + c * 16);
  }
}

template <int BM, int BN, int WGM, int WGN, bool FP8, bool SWIGLU, int OUT>
void launch(const GemmArgs& a, int64_t m_total, hipStream_t stream) {
  const int64_t mtiles = (m_total + (int64_t)a.n_groups * (BM - 1)) / BM;
  const int64_t grid = mtiles * a.n_tiles;
  if (grid <= 0) return;
  grouped_gemm_kernel<BM, BN, WGM, WGN, FP8, SWIGLU, OUT><<<(unsigned)grid, WGM * WGN * 64, 0, stream>>>(a);
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_grouped_gemm(const moe_gemm_desc* d, hipStream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(d != nullptr, MOE_ERR_NULL, "moe_grouped_gemm: desc is NULL");
  MOE_REQUIRE(d->w && d->group_offsets && (d->m_total == 0 || (d->a && d->out)), MOE_ERR_NULL,
              "moe_grouped_gemm: a, w, group_offsets and out are required");
  const bool fp8 = d->in_dtype == MOE_FP8_E4M3;
  MOE_REQUIRE(fp8 || d->in_dtype == MOE_BF16, MOE_ERR_DTYPE, "moe_grouped_gemm: in_dtype must be MOE_BF16 or MOE_FP8_E4M3");
  MOE_REQUIRE(d->epilogue == MOE_EPI_NONE || d->epilogue == MOE_EPI_SWIGLU, MOE_ERR_DTYPE,
              "moe_grouped_gemm: unknown epilogue %d", d->epilogue);
  const bool swiglu = d->epilogue == MOE_EPI_SWIGLU;
  MOE_REQUIRE(d->out_dtype == MOE_BF16 || d->out_dtype == MOE_F32 || d->out_dtype == MOE_FP8_E4M3, MOE_ERR_DTYPE,
              "moe_grouped_gemm: unknown out_dtype %d", d->out_dtype);
  MOE_REQUIRE(d->out_dtype != MOE_FP8_E4M3 || (fp8 && swiglu), MOE_ERR_DTYPE,
              "moe_grouped_gemm: an FP8 output needs FP8 inputs and the SwiGLU epilogue");
  MOE_REQUIRE(!(swiglu && d->out_dtype == MOE_F32), MOE_ERR_DTYPE, "moe_grouped_gemm: SwiGLU output must be bf16 or FP8");
  MOE_REQUIRE(d->n_groups >= 1 && d->n_groups <= 1024 && d->first_group >= 0, MOE_ERR_SHAPE,
              "moe_grouped_gemm: n_groups=%d first_group=%d", d->n_groups, d->first_group);
  MOE_REQUIRE(d->m_total >= 0 && d->m_total < ((int64_t)1 << 31), MOE_ERR_SHAPE, "moe_grouped_gemm: m_total=%lld",
              (long long)d->m_total);
  const int kstep_elems = fp8 ? 128 : 64;
  MOE_REQUIRE(d->K >= kstep_elems && d->K % kstep_elems == 0, MOE_ERR_SHAPE,
              "moe_grouped_gemm: K=%d must be a positive multiple of %d", d->K, kstep_elems);
  if (swiglu) {
    const int half_mult = fp8 ? 128 : 64;
    MOE_REQUIRE(d->N >= 2 * half_mult && (d->N / 2) % half_mult == 0 && d->N % 2 == 0, MOE_ERR_SHAPE,
                "moe_grouped_gemm: SwiGLU needs N/2 a positive multiple of %d (N=%d)", half_mult, d->N);
  } else {
    MOE_REQUIRE(d->N >= 128 && d->N % 128 == 0, MOE_ERR_SHAPE, "moe_grouped_gemm: N=%d must be a positive multiple of 128", d->N);
  }
  if (fp8) MOE_REQUIRE(d->a_scale && d->w_scale, MOE_ERR_NULL, "moe_grouped_gemm: FP8 inputs need a_scale and w_scale");
  if (d->out_dtype == MOE_FP8_E4M3) MOE_REQUIRE(d->out_scale, MOE_ERR_NULL, "moe_grouped_gemm: FP8 output needs out_scale");
  const int esz = fp8 ? 1 : 2;
  const int osz = d->out_dtype == MOE_F32 ? 4 : (d->out_dtype == MOE_BF16 ? 2 : 1);
  const int out_cols = swiglu ? d->N / 2 : d->N;
  MOE_REQUIRE(d->lda >= d->K && (d->lda * esz) % 16 == 0, MOE_ERR_ALIGN, "moe_grouped_gemm: lda=%lld", (long long)d->lda);
  MOE_REQUIRE(d->ldo >= out_cols && (d->ldo * osz) % 16 == 0, MOE_ERR_ALIGN, "moe_grouped_gemm: ldo=%lld", (long long)d->ldo);
  MOE_REQUIRE(aligned16(d->a) && aligned16(d->w) && aligned16(d->out), MOE_ERR_ALIGN,
              "moe_grouped_gemm: a, w and out must be 16-byte aligned");

  GemmArgs a;
  a.a = static_cast<const uint8_t*>(d->a);
  a.a_scale = d->a_scale;
  a.a_rows = d->a_rows;
  a.lda_b = d->lda * esz;
  a.w = static_cast<const uint8_t*>(d->w);
  a.w_scale = d->w_scale;
  a.offs = d->group_offsets + d->first_group;
  a.first_group = d->first_group;
  a.n_groups = d->n_groups;
  a.N = d->N;
  a.ksteps = d->K * esz / 128;
  a.ksb = d->K / 128;
  a.w_row_b = (int64_t)d->K * esz;
  a.out = static_cast<uint8_t*>(d->out);
  a.ldo_b = d->ldo * osz;
  a.out_scale = d->out_scale;
  a.out_scale_ld = out_cols / 128;

  if (!fp8) {
    a.n_tiles = swiglu ? (d->N / 2) / 64 : d->N / 128;
    if (swiglu) launch<128, 128, 2, 2, false, true, OUT_BF16>(a, d->m_total, stream);
    else if (d->out_dtype == MOE_BF16) launch<128, 128, 2, 2, false, false, OUT_BF16>(a, d->m_total, stream);
    else launch<128, 128, 2, 2, false, false, OUT_F32>(a, d->m_total, stream);
  } else {
    if (swiglu) {
      a.n_tiles = (d->N / 2) / 128;
      if (d->out_dtype == MOE_FP8_E4M3) launch<128, 256, 2, 4, true, true, OUT_FP8>(a, d->m_total, stream);
      else launch<128, 256, 2, 4, true, true, OUT_BF16>(a, d->m_total, stream);
    } else {
      a.n_tiles = d->N / 128;
      if (d->out_dtype == MOE_BF16) launch<128, 128, 2, 2, true, false, OUT_BF16>(a, d->m_total, stream);
      else launch<128, 128, 2, 2, true, false, OUT_F32>(a, d->m_total, stream);
    }
  }
  return check_launch("moe_grouped_gemm");
}
