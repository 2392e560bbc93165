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
//  * Power-of-two tile scales ("Vol.25 DeepSeek-V3の技術とその影響", "学習と推論の課題と解決
//    策": a tile shares one exponent; the report's "考察" asks for block scaling inside the
//    matrix unit): with E8M0 scale codes the block-scaled MFMA applies 2^(code - 127) per
//    operand row and 32-element K group itself, so every K slice accumulates straight into
//    the fp32 accumulator (no partial sums, no promotion FMAs).
//
// Design (CDNA4 first):
//  * Persistent workgroups, one per CU.  Each builds the per-expert tile table once (from the
//    device-side group offsets: no host synchronisation), then walks its share of the tiles.
//    Tiles are ordered (expert, column block, row block); each of the 8 XCDs gets a
//    contiguous range of that order and its workgroups stride through it in rounds, so the
//    activations of an expert and each weight block are fetched into that XCD's L2 once and
//    reused there (workgroup b runs on XCD b mod 8).  Reuse needs the workgroups of a round
//    to walk K together; left alone they drift apart by whole tiles over a launch, so in the
//    bf16 gate/up kernel with 128-row blocks each workgroup waits at the start of a round
//    until the XCD's other workgroups have finished the previous one (an arrival counter per
//    XCD in the caller's workspace; a workgroup arrives for each of its rounds, the last one
//    as it leaves; the wait is bounded, so it only ever costs time, and the last workgroup to
//    leave resets the counters for the next launch on that workspace).
//  * Row blocks of 128 rows (8 waves of 64x64), or 160 rows (8 waves of 80x64) for bf16
//    launches whose experts hold ~100-600 rows, where they need fewer row tiles per expert;
//    64 rows for decode-sized groups.
//  * Operands move HBM -> LDS with direct-to-LDS DMA (global_load_lds_dwordx4): each wave
//    instruction fills 8 rows x 128 bytes, the 16-byte chunks XOR-swizzled by (row & 7) so
//    the MFMA operand reads hit distinct banks.  A ring of STAGES K steps (128 bytes of K per
//    row: 64 bf16 or 128 E4M3) runs continuously across tile boundaries, with explicit
//    vmcnt waits and one barrier per step; a step's DMA instructions are spread over its
//    MFMAs (bf16: on a tile's last step they follow the tile's output stores); the gather indices of the next tile are fetched a whole tile ahead so the ring
//    never drains.
//  * A rows are gathered through the permutation (token of each sorted row); rows past an
//    expert's segment re-read its last row and are not stored.
//  * SwiGLU: the B tile holds BN/2 gate rows then the matching BN/2 up rows, and each wave
//    owns matching gate and up columns, so h is formed in registers.
//  * E4M3 products are formed W-first (D^T = W A^T): a lane's four results are four columns
//    of one token row, so one combined scale s_A * s_W promotes them; the scales of 8 K
//    blocks arrive by DMA into LDS beside the operands.
//  * The epilogue writes from registers (a tile's waves cover whole 128-byte lines, which
//    merge in L2); the fp8 output's per-row amax over its 128 columns is reduced across
//    waves in a small LDS array.
#include <math.h>

#include <type_traits>

#include "abi_common.h"
#include "device_common.h"

namespace moe {
namespace {

enum { OUT_BF16 = 0, OUT_F32 = 1, OUT_FP8 = 2 };
constexpr int kMaxGroups = 1024;
constexpr int kSyncSpins = 400;  // bound of a round wait: ~1 us per poll
// The workspace: round arrival counters of the 8 XCDs and an exit counter, zero between launches.
constexpr size_t kGemmWsBytes = 256;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// s_waitcnt through the builtin (so the compiler's own wait tracking sees it): gfx9
// encoding, vmcnt in bits [3:0] and [15:14], expcnt [6:4] = 7 and lgkmcnt [11:8] = 15 (no wait).
#define MOE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
#define MOE_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14))
// Workgroup barrier without the release fence of __syncthreads (which would wait for every
// outstanding DMA); LDS visibility of finished DMA is ensured by the vmcnt waits.
#define MOE_BARRIER()                \
  do {                               \
    MOE_WAIT_LGKM0();                \
    __builtin_amdgcn_s_barrier();    \
    asm volatile("" ::: "memory");   \
  } while (0)

struct GemmArgs {
  const uint8_t* a;
  const void* a_scale;   // f32 or E8M0 codes (u8)
  const int32_t* a_rows;
  int64_t lda_b;        // bytes per A row
  const uint8_t* w;
  const void* w_scale;
  const int32_t* offs;  // group_offsets + first_group (n_groups + 1 entries)
  int first_group;
  int n_groups;
  int N;                // rows of each W[g]
  int ksteps;           // number of 128-byte K steps
  int ksb;              // K / 128: scale columns (FP8)
  int64_t w_row_b;      // bytes per W row
  int out_cols;         // output columns (N, or N / 2 after SwiGLU)
  int n_tiles;          // output tiles along N
  uint8_t* out;
  int64_t ldo_b;        // bytes per output row
  void* out_scale;
  int out_scale_ld;
  int tail_first;       // first group (relative) writing the f32 tail output; n_groups if none
  uint8_t* out_tail;
  int64_t ldo_tail_b;   // bytes per tail output row
  unsigned int* sync;   // workspace: [8] round arrivals per XCD, [8] exit counter
  const int32_t* k_offs;  // per-group reduction lengths (k_offs[g + 1] - k_offs[g]), or null
  uint8_t* out_pre;       // SwiGLU: f32 gate | up products before the epilogue, or null
  int64_t ldo_pre_b;      // bytes per out_pre row
};

__device__ __forceinline__ float silu(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

struct TileInfo {
  int g;      // group index relative to first_group
  int nt;     // column block
  int row0;   // first global sorted row
  int nrows;  // valid rows (1..BM)
};

typedef __attribute__((address_space(4))) const int32_t cint32;

// A wave-uniform read of a group offset through the scalar cache (the offsets are not written
// by the kernel; scalar loads keep them off the vector-memory counter the DMA ring waits on).
__device__ __forceinline__ int load_offset(const int32_t* offs, int g) {
  return *(cint32*)(uintptr_t)(offs + __builtin_amdgcn_readfirstlane(g));
}

// Decode logical tile L (order: group, column block, row block; with band > 0, a group of more
// than `band` row blocks goes in bands of `band` row blocks, column blocks inside a band) from
// the LDS prefix table.
// Every caller walks its tiles in increasing L, so the search for the group (the largest g with
// tstart[g] <= L; then tstart[g + 1] > L, never an empty group) starts at the group of the
// caller's previous tile (cur, updated): a few steps forward, else a binary search over the rest.
template <int BM, bool BANDS>
__device__ __forceinline__ TileInfo decode_tile(int L, const int* tstart, int G, const int32_t* offs, int& cur,
                                                int band, int n_tiles) {
  int g = cur;
  for (int n = 0; n < 3 && g + 1 < G && __builtin_amdgcn_readfirstlane(tstart[g + 1]) <= L; ++n) ++g;
  if (g + 1 < G && __builtin_amdgcn_readfirstlane(tstart[g + 1]) <= L) {
    int lo = g, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tstart[mid] <= L) lo = mid;
      else hi = mid;
    }
    g = lo;
  }
  g = __builtin_amdgcn_readfirstlane(g);
  cur = g;
  const int local = L - tstart[g];
  const int m0 = load_offset(offs, g), m1 = load_offset(offs, g + 1);
  const int mt_g = (m1 - m0 + BM - 1) / BM;
  TileInfo t;
  t.g = g;
  t.nt = local / mt_g;
  int mt = local - t.nt * mt_g;
  if (BANDS && band > 0 && mt_g > band) {
    const int b = local / (band * n_tiles), r = local - b * band * n_tiles;
    const int rows_b = min(band, mt_g - b * band);  // the last band may be narrower
    t.nt = r / rows_b;
    mt = b * band + (r - t.nt * rows_b);
  }
  t.row0 = m0 + mt * BM;
  t.nrows = min(BM, m1 - t.row0);
  return t;
}

// FP8: 0 = bf16 inputs; 1 = E4M3 with f32 scales (promotion every K slice); 2 = E4M3 with
// E8M0 scales (applied by the matrix core).
// PRE: the training forward's SwiGLU launch, which also stores the gate | up products
// (out_pre); an instantiation of its own, so that the inference kernels carry none of its
// registers (the pointer kept live through the loop cost the E4M3 gate/up 3% in spilled
// scalar registers when it was a run-time option).
template <int BM, int BN, int WGM, int WGN, int STAGES, int FP8, bool SWIGLU, int OUT, bool PRE>
__global__ __launch_bounds__(WGM * WGN * 64) void grouped_gemm_kernel(GemmArgs p) {
  constexpr bool E8 = FP8 == 2;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM;  // rows per wave
  constexpr int WN = BN / WGN;  // W rows (output columns; gate+up for SwiGLU) per wave
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  // A DMA instruction q (rows 8q .. 8q + 7) is issued by wave q mod NW; with BM / 8 not a
  // multiple of NW the first waves issue one more (A_PW vs A_PW_MIN)
  constexpr int A_ROWS8 = BM / 8;
  constexpr int A_PW = (A_ROWS8 + NW - 1) / NW;     // A DMA instructions per wave per stage (at most)
  constexpr int A_PW_MIN = A_ROWS8 / NW;            // ... (at least)
  constexpr int B_PW = BN / 8 / NW;               // B DMA instructions per wave per stage
  // Scales arrive in chunks of SC_CH K blocks, one 4-byte DMA per lane, into one of SC_NB LDS
  // buffers in turn: BM * SC_CH A scales (SC_PW instructions per wave) and, from wave 0, the
  // two weight-block scales of the tile's columns for the same K blocks (SC_WS floats).  A
  // chunk's DMA is issued STAGES - 1 steps before its first step and overwrites the chunk
  // SC_NB earlier, whose last step is at least SC_NB steps back: SC_NB = STAGES keeps it behind
  // the barrier of the issuing step.  E8M0 codes are bytes: a chunk then spans 256 * NW / BM
  // K blocks, so that its A codes (one dword = 4 K blocks of a row) are one DMA per lane.
  constexpr int SC_CH = E8 ? 256 * NW / BM : 8;
  constexpr int SC_NB = STAGES;
  constexpr int SC_DW = E8 ? BM * SC_CH / 4 : BM * SC_CH;  // dwords of A scales per chunk
  constexpr int SC_PW = FP8 ? SC_DW / 64 / NW : 0;
  constexpr int SC_WS = E8 ? SC_CH / 2 : 2 * SC_CH;  // weight-scale dwords: [2 blocks][SC_CH K blocks]
  constexpr int SC_BUF = SC_DW + SC_WS;              // dwords per chunk buffer
  constexpr int OC = SWIGLU ? BN / 2 : BN;
  // data DMA instructions per wave per stage: L_ISSUE at most, L_STAGE at least (the vmcnt
  // waits allow L_STAGE later instructions in flight; a wave that issued more only waits
  // longer; a scale chunk adds SC_PW)
  constexpr int L_ISSUE = A_PW + B_PW;
  constexpr int L_STAGE = A_PW_MIN + B_PW;
  static_assert(A_ROWS8 * 8 == BM && B_PW * 8 * NW == BN && A_PW_MIN >= 1, "DMA rows must split over waves");
  static_assert(!FP8 || (SC_PW >= 1 && SC_PW * 64 * NW == SC_DW && A_PW == A_PW_MIN),
                "scale chunk DMA must split evenly over waves");
  static_assert(!E8 || (SC_CH % 4 == 0 && SC_WS <= 64), "E8M0 chunks hold whole dwords of 4 K blocks");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(!SWIGLU || TN % 2 == 0, "SwiGLU waves need matching gate and up tiles");
  static_assert(OUT != OUT_FP8 || (FP8 && SWIGLU && OC == 128), "fp8 output = one 1x128 tile per row");
  static_assert(!FP8 || (SWIGLU ? WN / 2 <= 128 : WN <= 128), "a wave must sit inside one 128-row scale block");
  static_assert(!FP8 || (BN == 256 && TM == 4), "E4M3 tiles: two 128-row weight blocks, 4 row tiles per wave");
  static_assert(STAGES == 2 || STAGES == 3, "the ring has two or three slots");
  // Round synchronisation pays where a round's workgroups share most of their operands and
  // the launch is bandwidth-bound: the bf16 gate/up projection with 128-row blocks (the
  // bf16 T = 4096 routing: 3.99 -> 3.69 ms), where an expert's rows span two blocks that
  // share its weights.  Elsewhere it measured neutral or slower (160-row blocks, which hold
  // most experts in one block: 3.33 -> 3.11 ms without it; the down projections, whose
  // rounds span several experts; the E4M3 kernels; decode-sized blocks), so it is compiled
  // out there.
  constexpr bool kRoundSync = SWIGLU && !FP8 && BM == 128;
  static_assert(L_STAGE * (STAGES - 2) <= 63, "vmcnt budget");

  // one LDS array per ring slot: distinct objects, so the compiler can tell the DMA target of
  // a step apart from the slot being read and adds no waits of its own
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[STAGES > 2 ? STAGE : 16];
  // scales: SC_NB chunk buffers, used in turn over the sequence of chunks this workgroup loads
  __shared__ __attribute__((aligned(16))) float s_sc[FP8 ? SC_NB * SC_BUF : 1];
  __shared__ float s_red[OUT == OUT_FP8 ? WGN * BM : 1];
  // tile prefix table (G + 1 ints), sized at launch
  extern __shared__ int s_tstart[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave - wm * WGN;
  const int G = p.n_groups;

  // ---- tile table: exclusive prefix of (row blocks x column blocks) over the groups ----
  if (wave == 0) {
    const int per = (G + 63) >> 6;
    const int g0 = min(G, lane * per), g1 = min(G, g0 + per);
    int local = 0;
    for (int g = g0; g < g1; ++g) local += (p.offs[g + 1] - p.offs[g] + BM - 1) / BM * p.n_tiles;
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    int run = incl - local;
    for (int g = g0; g < g1; ++g) {
      s_tstart[g] = run;
      run += (p.offs[g + 1] - p.offs[g] + BM - 1) / BM * p.n_tiles;
    }
    if (lane == 63) s_tstart[G] = incl;
  }
  __syncthreads();
  const int total = s_tstart[G];
  const int n_xcd = gridDim.x >= 8 ? 8 : 1;
  const int xcd = blockIdx.x % n_xcd, slot = blockIdx.x / n_xcd, per_xcd = gridDim.x / n_xcd;
  const int t_begin = (int)((int64_t)total * xcd / n_xcd), t_end = (int)((int64_t)total * (xcd + 1) / n_xcd);
  const int n_my = t_end - t_begin > slot ? (t_end - t_begin - slot + per_xcd - 1) / per_xcd : 0;
  const int ksteps = p.ksteps;
  // Ragged reduction (f32 outputs without SwiGLU, f32 scales): with k_offs set, the tiles of
  // group g run only the K steps that cover its first k_offs[g + 1] - k_offs[g] elements (at
  // least one step), so a weight gradient over zero-padded expert segments skips the padding
  // beyond each expert's own length.  The walk over a workgroup's steps then keeps its own
  // (tile, step) counters instead of dividing by a common step count.
  constexpr bool kRag = OUT == OUT_F32 && !SWIGLU && !E8;
  constexpr int kGran = FP8 ? 128 : 64;  // K elements per step
  // Tile order of the E4M3 weight gradients (ragged launches with 16+ column blocks, i.e. the
  // gate/up weights' gradient: 4096 rows x 28 column blocks per expert): bands of two row
  // blocks, so that a round of an XCD's 32 workgroups covers 2 row blocks x 16 column blocks
  // rather than 32 row blocks of one column block; measured 13.0 -> 10.6 ms at T = 16384.  The
  // narrower down-projection gradient (8 column blocks) and the bf16 launches measured equal
  // or slower with bands, so they keep the plain order.
  constexpr bool kBands = kRag && FP8 == 1;
  const int band = (kBands && p.k_offs && p.n_tiles >= 16) ? 2 : 0;
  auto group_ksteps = [&](int g) {
    if constexpr (kRag) {
      if (p.k_offs) {
        const int len = load_offset(p.k_offs, g + 1) - load_offset(p.k_offs, g);
        return len <= 0 ? 1 : min(ksteps, (len - 1) / kGran + 1);
      }
    }
    return ksteps;
  };
  int total_steps = n_my * ksteps;
  if constexpr (kRag) {
    if (p.k_offs) {
      total_steps = 0;
      int cur = 0;
#pragma unroll 1
      for (int q = 0; q < n_my; ++q)
        total_steps +=
            group_ksteps(decode_tile<BM, kBands>(t_begin + slot + q * per_xcd, s_tstart, G, p.offs, cur, band, p.n_tiles).g);
    }
  }
  // arrivals the XCD's counter holds once every workgroup with a round-r tile finished it,
  // summed over rounds r < q
  const int xr = t_end - t_begin;
  auto round_target = [&](int q) {
    unsigned int tgt = 0;
#pragma unroll 1
    for (int r = 0; r < q; ++r) tgt += (unsigned int)max(0, min(per_xcd, xr - r * per_xcd));
    return tgt;
  };
  // A workgroup arrives for round r - 1 as it starts round r, and for its last round as it
  // leaves, so the counter of an XCD reaches round_target(q) once every workgroup with a tile
  // in rounds < q has finished it.  The last workgroup to leave resets the counters.
  auto leave = [&]() {
    if constexpr (kRoundSync) {
      if (tid == 0) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (n_my > 0) __hip_atomic_fetch_add(&p.sync[xcd], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned int prev = __hip_atomic_fetch_add(&p.sync[8], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == gridDim.x - 1) {  // last workgroup out: reset for the next launch
          for (int x = 0; x < 8; ++x) __hip_atomic_store(&p.sync[x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&p.sync[8], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };
  if (total_steps == 0) {
    leave();
    return;
  }

  // ---- loader state ----
  const int cch = lane & 7;
  const int lrow = lane >> 3;  // row within an 8-row DMA instruction
  const uint8_t* a_ptr[A_PW];
  int a_nxt[A_PW];
  int b_off[B_PW];
  const float* s_ptr[SC_PW > 0 ? SC_PW : 1];     // f32 scale rows
  const uint8_t* s8_ptr[SC_PW > 0 ? SC_PW : 1];  // E8M0 code rows
  int s_nxt[SC_PW > 0 ? SC_PW : 1];
  // A-scale chunk layout: [BM / 4 row groups][SC_CH K blocks, swizzled][4 rows].  Row group
  // g = wm * 16 + lr holds rows wm * WM + i * 16 + lr (i = 0..3), the four rows whose products
  // one lane accumulates, so a K step reads its four scales with one 16-byte LDS read; the K
  // block slot is XORed with ((g >> 1) & 7), which puts the 16 row groups of a read (two per
  // 256-byte bank row) on distinct banks.
  // DMA lane (instruction q, lane l) fills dword d = q * 64 + l: row group d / 32, slot
  // (d / 4) % 8, row index d % 4; its 8 consecutive slots of a row read 32 contiguous bytes.
  static_assert(E8 || SC_CH == 8, "the scale swizzle assumes 8 K blocks per chunk");
  int sc_col[SC_PW > 0 ? SC_PW : 1];  // K block (within a chunk) that each scale DMA of this lane fetches
  int sc_row[SC_PW > 0 ? SC_PW : 1];  // tile row that each scale DMA of this lane fetches
  // E8M0 chunk layout: [BM / 4 row groups][SC_CH / 4 dwords of 4 K blocks][4 rows], so a K
  // step reads the codes of a lane's four rows with one 16-byte read; DMA dword d holds row
  // index d % 4 of group d / SC_CH, K blocks 4 * ((d / 4) % (SC_CH / 4)) .. + 3.
#pragma unroll
  for (int i = 0; i < SC_PW; ++i) {
    const int d = (wave * SC_PW + i) * 64 + lane;
    if constexpr (E8) {
      const int grp = d / SC_CH;
      sc_col[i] = 4 * ((d >> 2) % (SC_CH / 4));
      sc_row[i] = (grp >> 4) * WM + (d & 3) * 16 + (grp & 15);
    } else {
      const int grp = d >> 5;
      sc_col[i] = ((d >> 2) & 7) ^ ((grp >> 1) & 7);
      sc_row[i] = (grp >> 4) * WM + (d & 3) * 16 + (grp & 15);
    }
  }
  // weight-block scales (lanes 0..15 of wave 0): lane l loads K block l >> 1 of block l & 1 --
  // the gate and up blocks under SwiGLU, else the tile's two 128-column blocks
  const float* w_sc_ptr = static_cast<const float*>(p.w_scale);
  // E8M0: lane l < SC_WS loads the dword of K blocks 4 * (l % (SC_CH / 4)) .. + 3 of weight
  // block l / (SC_CH / 4) (gate / up under SwiGLU, else the tile's two 128-column blocks)
  const uint8_t* w_sc8 = static_cast<const uint8_t*>(p.w_scale);
  const int w_kq4 = 4 * (lane % (SC_CH / 4 > 0 ? SC_CH / 4 : 1));
  int sc_issue = 0;                 // buffer of the next chunk to issue
  int lq = -1;  // index (in this workgroup's list) of the tile being loaded
  const uint8_t* wbase = p.w;

  // tile q of this workgroup; the three walks over the tiles (weight rows of the batch being
  // loaded, gather rows one tile ahead, the tile being computed) keep their own search cursors
  int cur_b = 0, cur_r = 0, cur_c = 0;
  auto tile_of = [&](int q, int& cur) {
    return decode_tile<BM, kBands>(t_begin + slot + q * per_xcd, s_tstart, G, p.offs, cur, band, p.n_tiles);
  };
  // gather sources of a tile's rows (global loads whose values are used one tile later)
  auto fetch_rows = [&](const TileInfo& t, int* dst, int* sdst) {
#pragma unroll
    for (int i = 0; i < A_PW; ++i) {
      const int q = wave + NW * i;
      const int rr = 8 * min(q, A_ROWS8 - 1) + lrow;
      const int r = t.row0 + min(rr, t.nrows - 1);
      dst[i] = p.a_rows ? p.a_rows[r] : r;
    }
#pragma unroll
    for (int i = 0; i < SC_PW; ++i) {
      const int r = t.row0 + min(sc_row[i], t.nrows - 1);
      sdst[i] = p.a_rows ? p.a_rows[r] : r;
    }
  };
  auto set_rows = [&](const int* src, const int* ssrc) {
#pragma unroll
    for (int i = 0; i < A_PW; ++i) {
      const int rr = 8 * (wave + NW * i) + lrow;
      a_ptr[i] = p.a + (int64_t)src[i] * p.lda_b + ((cch ^ (rr & 7)) << 4);
    }
#pragma unroll
    for (int i = 0; i < SC_PW; ++i) {
      if constexpr (E8) s8_ptr[i] = static_cast<const uint8_t*>(p.a_scale) + (int64_t)ssrc[i] * p.ksb;
      else s_ptr[i] = static_cast<const float*>(p.a_scale) + (int64_t)ssrc[i] * p.ksb;
    }
  };
  auto set_b = [&](const TileInfo& t) {
#pragma unroll
    for (int i = 0; i < B_PW; ++i) {
      const int rr = 8 * (wave * B_PW + i) + lrow;
      int n;
      if (SWIGLU) n = (rr < BN / 2) ? t.nt * (BN / 2) + rr : p.N / 2 + t.nt * (BN / 2) + (rr - BN / 2);
      else n = t.nt * BN + rr;
      b_off[i] = (int)(n * p.w_row_b) + ((cch ^ (rr & 7)) << 4);
    }
    wbase = p.w + (int64_t)(p.first_group + t.g) * p.N * p.w_row_b;
    if constexpr (E8) {
      const int sel = (lane / (SC_CH / 4)) & 1;
      const int nblk = SWIGLU ? (sel ? p.N / 2 + t.nt * (BN / 2) : t.nt * (BN / 2)) / 128 : (t.nt * BN) / 128 + sel;
      w_sc8 = static_cast<const uint8_t*>(p.w_scale) + ((int64_t)(p.first_group + t.g) * (p.N / 128) + nblk) * p.ksb;
    } else if constexpr (FP8 != 0) {
      const int sel = lane & 1;
      const int nblk = SWIGLU ? (sel ? p.N / 2 + t.nt * (BN / 2) : t.nt * (BN / 2)) / 128 : (t.nt * BN) / 128 + sel;
      w_sc_ptr = static_cast<const float*>(p.w_scale) + ((int64_t)(p.first_group + t.g) * (p.N / 128) + nblk) * p.ksb +
                 ((lane & 15) >> 1);
    }
  };
  // issue the DMA of global step js (clamped to the last step: every step issues one batch,
  // so the number of batches in flight is constant) into ring slot SL
  int dma_kt = 0;            // K step of the batch being issued
  bool dma_scales = false;   // the batch starts a scale chunk
  int ld_js = -1, ld_q = -1, ld_kt = 0, ld_ks = 0;  // ragged: step, tile, K step, tile's K steps
  // tile bookkeeping for the batch of global step js (clamped to the last step: every step
  // issues one batch, so the number of batches in flight is constant)
  auto issue_prep = [&](int js) __attribute__((always_inline)) {
    const bool past_end = js >= total_steps;
    js = min(js, total_steps - 1);
    int q, kt;
    if constexpr (kRag) {
      if (js != ld_js) {  // the next step (the calls advance one step at a time)
        ld_js = js;
        if (++ld_kt >= ld_ks) {
          ++ld_q;
          ld_kt = 0;
        }
      }
      q = ld_q;
      kt = ld_kt;
    } else {
      q = js / ksteps;
      kt = js - q * ksteps;
    }
    if (q != lq) {  // entering a new tile: its rows were fetched one tile earlier
      const TileInfo tb = tile_of(q, cur_b);
      set_b(tb);
      if constexpr (kRag) ld_ks = group_ksteps(tb.g);
      if (q > 0) set_rows(a_nxt, s_nxt);
      if (q + 1 < n_my) fetch_rows(tile_of(q + 1, cur_r), a_nxt, s_nxt);
      lq = q;
    }
    dma_kt = kt;
    dma_scales = FP8 != 0 && !past_end && kt % SC_CH == 0;
  };
  // data DMA instruction k (0 .. L_ISSUE - 1: A rows, then B rows) of the prepared batch into
  // ring slot SL
  auto issue_one = [&](auto slot_c, int k) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    uint8_t* st = SL == 0 ? slot0 : (SL == 1 ? slot1 : slot2);
    if (k < A_PW) {
      const int q = wave + NW * k;
      if (A_PW == A_PW_MIN || q < A_ROWS8)
        __builtin_amdgcn_global_load_lds((glb_void*)(a_ptr[k] + dma_kt * 128), (lds_void*)(st + q * 1024), 16, 0, 0);
    } else {
      const int i = k - A_PW;
      __builtin_amdgcn_global_load_lds((glb_void*)(wbase + dma_kt * 128 + (uint32_t)b_off[i]),
                                       (lds_void*)(st + A_BYTES + (wave * B_PW + i) * 1024), 16, 0, 0);
    }
  };
  // the scales of K blocks [kt, kt + SC_CH) of the tile's rows and weight blocks (clamped to
  // the last block), when the prepared batch starts a chunk
  auto issue_scales = [&]() __attribute__((always_inline)) {
    if (dma_scales) {
      const int kt = dma_kt;
      float* sc = s_sc + sc_issue * SC_BUF;
      if constexpr (E8) {  // dwords of 4 codes; the last dword of a row is the clamp (ksb % 4 == 0)
#pragma unroll
        for (int i = 0; i < SC_PW; ++i)
          __builtin_amdgcn_global_load_lds((glb_void*)(s8_ptr[i] + min(kt + sc_col[i], p.ksb - 4)),
                                           (lds_void*)(sc + (wave * SC_PW + i) * 64), 4, 0, 0);
        if (wave == 0 && lane < SC_WS)
          __builtin_amdgcn_global_load_lds((glb_void*)(w_sc8 + min(kt + w_kq4, p.ksb - 4)), (lds_void*)(sc + SC_DW), 4,
                                           0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < SC_PW; ++i)
          __builtin_amdgcn_global_load_lds((glb_void*)(s_ptr[i] + min(kt + sc_col[i], p.ksb - 1)),
                                           (lds_void*)(sc + (wave * SC_PW + i) * 64), 4, 0, 0);
        if (wave == 0 && lane < SC_WS)
          __builtin_amdgcn_global_load_lds((glb_void*)(w_sc_ptr + min(kt, p.ksb - 1 - ((lane & 15) >> 1))),
                                           (lds_void*)(sc + BM * SC_CH), 4, 0, 0);
      }
      sc_issue = sc_issue + 1 == SC_NB ? 0 : sc_issue + 1;
    }
  };
  // the whole batch at once (the ring's first steps)
  auto issue = [&](auto slot_c, int js) __attribute__((always_inline)) {
    issue_prep(js);
#pragma unroll
    for (int k = 0; k < L_ISSUE; ++k) issue_one(slot_c, k);
    issue_scales();
  };
  // Inside a step the batch's instructions are spread over the MFMA sequence (instruction k
  // after MFMA dma_pos(k, n) of n), each fenced so the compiler keeps it there: a wave that
  // issued its whole batch at once would stall until the texture unit had taken it
  // (~16 cycles per 1 KB instruction per CU), while spread out they queue behind nothing.
  // bf16: the last step of a tile issues its batch after the tile's output stores instead.  A
  // wave's vector-memory instructions enter the texture unit in order, so stores issued right
  // behind a batch of 1 KB DMA instructions wait for it (~4 us per tile at 80 stores per wave);
  // with the batch behind them the ring, two steps deep, still covers it (T = 4096: gate/up
  // -2.7%, down -1.4%, backward -3.8%).  The E4M3 tiles store a quarter as many instructions
  // and lose more than they gain (down +2%), so they keep the batch spread over the products.
  bool dma_now = true;
  auto dma_in = [&](auto slot_c, int t, int n) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < L_ISSUE; ++k)
      if (t == (k + 1) * n / (L_ISSUE + 1) && (FP8 || dma_now)) {
        __builtin_amdgcn_sched_barrier(0);
        issue_one(slot_c, k);
        __builtin_amdgcn_sched_barrier(0);
      }
  };


  // rows of the first tile (the ring is empty, so waiting for them costs nothing)
  {
    int src0[A_PW];
    int ssrc0[SC_PW > 0 ? SC_PW : 1];
    fetch_rows(tile_of(0, cur_r), src0, ssrc0);
    set_rows(src0, ssrc0);
  }
  issue(std::integral_constant<int, 0>(), 0);
  if constexpr (STAGES > 2) issue(std::integral_constant<int, 1>(), 1);

  // ---- compute state ----
  const int lr = lane & 15, lg = lane >> 4;
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  TileInfo ct = tile_of(0, cur_c);
  int c_q = 0, c_kt = 0, c_ks = group_ksteps(ct.g);  // ragged: tile, K step, tile's K steps
  // operand reads: row & 7 = lr & 7 for every row a lane reads (tile offsets are multiples of
  // 16), so its two swizzled 16-byte chunks (lg and lg + 4) sit at fixed byte offsets lo / hi
  // from the row start and every read is one base register plus a constant
  const int sw_lo = (lg ^ (lr & 7)) << 4, sw_hi = sw_lo ^ 64;
  const int fa_lo = (wm * WM + lr) * 128 + sw_lo, fa_hi = (wm * WM + lr) * 128 + sw_hi;
  const int fb_row = SWIGLU ? wn * (WN / 2) + lr : wn * WN + lr;
  const int fb_lo = fb_row * 128 + sw_lo, fb_hi = fb_row * 128 + sw_hi;
  const int fs_off = (wm * 16 + lr) * (SC_CH * 4);  // this lane's scale row group (f32)
  const int fs8_off = (wm * 16 + lr) * SC_CH;       // ... (E8M0: dwords)
  const int base_row = load_offset(p.offs, 0);
  const int tail_row = load_offset(p.offs, min(p.tail_first, G));
  int sc_use = 0;  // buffer of the chunk being consumed (same sequence as sc_issue)

  constexpr int TO = SWIGLU ? TN / 2 : TN;  // output tiles per wave row block

  // ---- E4M3 K step, in two halves: operand + scale reads, then the products ----
  // A lane's 32 bytes of the 128-element K slice are chunks lg and lg + 4 (the same K
  // permutation for A and B leaves the product unchanged); each read then covers the 16
  // lanes' rows at distinct swizzled chunks and hits distinct banks.  The scales of the K
  // block: s_A of the lane's four rows (one 16-byte read) and the two weight-block scales
  // (one broadcast read), combined into s_A * s_W per row tile.
  auto fp8_read = [&](const uint8_t* As, int kt, int tks, i32x8(&af)[TM], i32x8(&bfr)[TN], float(&s0)[TM],
                      float(&s1)[TM]) __attribute__((always_inline)) {
    const uint8_t* Bs = As + A_BYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const u32x4 lo = *(const u32x4*)(As + fa_lo + i * 16 * 128);
      const u32x4 hi = *(const u32x4*)(As + fa_hi + i * 16 * 128);
      af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) {
      const int ro = (SWIGLU && jj >= TN / 2 ? BN / 2 + (jj - TN / 2) * 16 : jj * 16) * 128;
      const u32x4 lo = *(const u32x4*)(Bs + fb_lo + ro);
      const u32x4 hi = *(const u32x4*)(Bs + fb_hi + ro);
      bfr[jj] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    const int kc = kt % SC_CH;
    const float* scb = s_sc + sc_use * SC_BUF;
    const f32x4 sa = *(const f32x4*)(scb + fs_off + ((kc ^ ((lr >> 1) & 7)) << 2));
    const float* swp = scb + BM * SC_CH + 2 * kc;
    const float sw0 = SWIGLU || (wn * WN) / 128 == 0 ? swp[0] : swp[1], sw1 = swp[1];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      s0[i] = sa[i] * sw0;
      s1[i] = SWIGLU ? sa[i] * sw1 : s0[i];
    }
    if (kc == SC_CH - 1 || kt == tks - 1) sc_use = sc_use + 1 == SC_NB ? 0 : sc_use + 1;  // chunk done
  };
  // Products with W as the first operand: a lane's four results of tile (i, jj) are columns
  // lg * 4 .. lg * 4 + 3 of row lr, so one combined scale covers them.  Every tile's partial
  // sum gets its own registers and its promotion (fp32 FMA into the accumulator) trails the
  // matrix core by two tiles, so MFMAs issue back to back while the VALU promotes.
  auto fp8_math = [&](auto slot_c, const i32x8(&af)[TM], const i32x8(&bfr)[TN], const float(&s0)[TM],
                      const float(&s1)[TM]) __attribute__((always_inline)) {
    constexpr int NT = TM * TN;
    f32x4 pq[NT];
#pragma unroll
    for (int t = 0; t < NT + 2; ++t) {
      if (t < NT) {
        pq[t] = mfma_fp8(bfr[t % TN], af[t / TN], f32x4{0.f, 0.f, 0.f, 0.f});
        dma_in(slot_c, t, NT);
      }
      if (t >= 2) {
        const int u = t - 2, i = u / TN, jj = u % TN;
        const float sc = SWIGLU && jj >= TN / 2 ? s1[i] : s0[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][jj][r] = fmaf(pq[u][r], sc, acc[i][jj][r]);
      }
    }
  };

  // ---- E8M0 K step: the same operand reads, the codes of the lane's four rows (one 16-byte
  // read, byte kc % 4 of each dword) and of the two weight blocks; every product goes straight
  // into its accumulator with the codes as the MFMA's block scales ----
  auto e8_read = [&](const uint8_t* As, int kt, int tks, i32x8(&af)[TM], i32x8(&bfr)[TN], int(&sa)[TM], int& sw0,
                     int& sw1) __attribute__((always_inline)) {
    const uint8_t* Bs = As + A_BYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const u32x4 lo = *(const u32x4*)(As + fa_lo + i * 16 * 128);
      const u32x4 hi = *(const u32x4*)(As + fa_hi + i * 16 * 128);
      af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) {
      const int ro = (SWIGLU && jj >= TN / 2 ? BN / 2 + (jj - TN / 2) * 16 : jj * 16) * 128;
      const u32x4 lo = *(const u32x4*)(Bs + fb_lo + ro);
      const u32x4 hi = *(const u32x4*)(Bs + fb_hi + ro);
      bfr[jj] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    const int kc = kt % SC_CH;
    const uint32_t* scb = reinterpret_cast<const uint32_t*>(s_sc) + sc_use * SC_BUF;
    const u32x4 d4 = *(const u32x4*)(scb + fs8_off + ((kc >> 2) << 2));
    const int sh = (kc & 3) << 3;
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = (int)((d4[i] >> sh) & 255u);
    const uint32_t* swp = scb + SC_DW + (kc >> 2);
    const uint32_t w0 = swp[0], w1 = swp[SC_CH / 4];
    sw0 = (int)(((SWIGLU || (wn * WN) / 128 == 0 ? w0 : w1) >> sh) & 255u);
    sw1 = (int)((w1 >> sh) & 255u);
    if (kc == SC_CH - 1 || kt == tks - 1) sc_use = sc_use + 1 == SC_NB ? 0 : sc_use + 1;  // chunk done
  };
  auto e8_math = [&](auto slot_c, const i32x8(&af)[TM], const i32x8(&bfr)[TN], const int(&sa)[TM], int sw0, int sw1)
      __attribute__((always_inline)) {
    constexpr int NT = TM * TN;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = t / TN, jj = t % TN;
      acc[i][jj] = mfma_fp8_e8m0(bfr[jj], af[i], acc[i][jj], SWIGLU && jj >= TN / 2 ? sw1 : sw0, sa[i]);
      dma_in(slot_c, t, NT);
    }
  };

  // ---- SwiGLU with out_pre: the gate and up products themselves (a | c, the epilogue's inputs)
  // also stored, f32 rows of N columns (gate in [0, N/2), up in [N/2, N)), for a backward pass
  // that would otherwise recompute them with a second gate/up GEMM ----
  auto epi_preact = [&](const TileInfo& et) __attribute__((always_inline)) {
    if constexpr (SWIGLU) {
      const int64_t orow0 = (int64_t)(et.row0 - base_row);
      const int half = p.N / 2;
      if constexpr (FP8) {  // lane: row wm * WM + i * 16 + lr, columns c0 + jj * 16 + 0..3
        const int c0 = et.nt * OC + wn * (WN / 2) + lg * 4;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int m = wm * WM + i * 16 + lr;
          if (m >= et.nrows) continue;
          float* prow = reinterpret_cast<float*>(p.out_pre + (orow0 + m) * p.ldo_pre_b);
#pragma unroll
          for (int jj = 0; jj < TO; ++jj) {
            *reinterpret_cast<f32x4*>(prow + c0 + jj * 16) = acc[i][jj];
            *reinterpret_cast<f32x4*>(prow + half + c0 + jj * 16) = acc[i][jj + TO];
          }
        }
      } else {  // lane: rows wm * WM + i * 16 + lg * 4 + r, column c0 + jj * 16
        const int c0 = et.nt * OC + wn * (WN / 2) + lr;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = wm * WM + i * 16 + lg * 4 + r;
            if (m >= et.nrows) continue;
            float* prow = reinterpret_cast<float*>(p.out_pre + (orow0 + m) * p.ldo_pre_b);
#pragma unroll
            for (int jj = 0; jj < TO; ++jj) {
              prow[c0 + jj * 16] = acc[i][jj][r];
              prow[half + c0 + jj * 16] = acc[i][jj + TO][r];
            }
          }
      }
    }
  };

  // ---- epilogue of a tile: values (SwiGLU applied; the accumulators restart at zero), the
  // per-row amax of an E4M3 output into s_red, then the stores ----
  auto epi_values = [&](float(&v)[TM][TO][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TO; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[i][jj][r] = SWIGLU ? silu(acc[i][jj][r]) * acc[i][jj + TO][r] : acc[i][jj][r];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // E4M3 layout (FP8): lane holds row wm * WM + i * 16 + lr, columns col_w + jj * 16 + 0..3;
  // bf16 layout: rows wm * WM + i * 16 + lg * 4 + r, column col_w + jj * 16
  auto epi_reduce = [&](const float(&v)[TM][TO][4]) __attribute__((always_inline)) {
    if constexpr (OUT == OUT_FP8) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        float mx = 0.f;
#pragma unroll
        for (int jj = 0; jj < TO; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(v[i][jj][r]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        if (lg == 0) s_red[wn * BM + wm * WM + i * 16 + lr] = mx;  // the 4 lanes of the row agree
      }
    }
  };
  auto epi_store = [&](const float(&v)[TM][TO][4], const TileInfo& et) __attribute__((always_inline)) {
    const int64_t orow0 = (int64_t)(et.row0 - base_row);
    const bool tail = OUT == OUT_BF16 && !SWIGLU && et.g >= p.tail_first;  // split output: f32 tail rows
    if constexpr (FP8) {
      const int c0 = et.nt * OC + (SWIGLU ? wn * (WN / 2) : wn * WN) + lg * 4;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = wm * WM + i * 16 + lr;
        if (OUT == OUT_FP8) {
          float amax = 0.f;
#pragma unroll
          for (int q = 0; q < WGN; ++q) amax = fmaxf(amax, s_red[q * BM + m]);
          if constexpr (E8) {  // power-of-two scale: exact products by 2^-k
            const int k = e8m0_exponent(amax);
            const float inv = pow2f(-k);
            if (m < et.nrows) {
              uint8_t* orow = p.out + (orow0 + m) * p.ldo_b;
#pragma unroll
              for (int jj = 0; jj < TO; ++jj) {
                uint32_t w4 = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) w4 |= f32_to_e4m3(v[i][jj][r] * inv) << (8 * r);
                *reinterpret_cast<uint32_t*>(orow + c0 + jj * 16) = w4;
              }
              if (wn == 0 && lg == 0)
                static_cast<uint8_t*>(p.out_scale)[(orow0 + m) * p.out_scale_ld + et.nt] = (uint8_t)(k + 127);
            }
          } else {
            const float s = (amax == 0.f) ? 1.0f : amax / 448.0f;
            const float rs = recip_refined(s);
            if (m < et.nrows) {
              uint8_t* orow = p.out + (orow0 + m) * p.ldo_b;
#pragma unroll
              for (int jj = 0; jj < TO; ++jj) {
                uint32_t w4 = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) w4 |= f32_to_e4m3(quotient(v[i][jj][r], s, rs)) << (8 * r);
                *reinterpret_cast<uint32_t*>(orow + c0 + jj * 16) = w4;
              }
              if (wn == 0 && lg == 0) static_cast<float*>(p.out_scale)[(orow0 + m) * p.out_scale_ld + et.nt] = s;
            }
          }
        } else if (m < et.nrows) {
          if (tail) {
            float* trow = reinterpret_cast<float*>(p.out_tail + (int64_t)(et.row0 - tail_row + m) * p.ldo_tail_b);
#pragma unroll
            for (int jj = 0; jj < TO; ++jj)
              *reinterpret_cast<f32x4*>(trow + c0 + jj * 16) = f32x4{v[i][jj][0], v[i][jj][1], v[i][jj][2], v[i][jj][3]};
          } else {
            uint8_t* orow = p.out + (orow0 + m) * p.ldo_b;
#pragma unroll
            for (int jj = 0; jj < TO; ++jj) {
              if (OUT == OUT_F32)
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(orow) + c0 + jj * 16) =
                    f32x4{v[i][jj][0], v[i][jj][1], v[i][jj][2], v[i][jj][3]};
              else
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(orow) + c0 + jj * 16) =
                    u32x2{f32_to_bf16_rne(v[i][jj][0]) | (f32_to_bf16_rne(v[i][jj][1]) << 16),
                          f32_to_bf16_rne(v[i][jj][2]) | (f32_to_bf16_rne(v[i][jj][3]) << 16)};
            }
          }
        }
      }
    } else {
      const int c0 = et.nt * OC + (SWIGLU ? wn * (WN / 2) : wn * WN) + lr;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = wm * WM + i * 16 + lg * 4 + r;
          if (m >= et.nrows) continue;
          if (tail) {
            float* trow = reinterpret_cast<float*>(p.out_tail + (int64_t)(et.row0 - tail_row + m) * p.ldo_tail_b);
#pragma unroll
            for (int jj = 0; jj < TO; ++jj) trow[c0 + jj * 16] = v[i][jj][r];
          } else {
            uint8_t* orow = p.out + (orow0 + m) * p.ldo_b;
#pragma unroll
            for (int jj = 0; jj < TO; ++jj) {
              const int c = c0 + jj * 16;
              if (OUT == OUT_F32) reinterpret_cast<float*>(orow)[c] = v[i][jj][r];
              else reinterpret_cast<uint16_t*>(orow)[c] = (uint16_t)f32_to_bf16_rne(v[i][jj][r]);
            }
          }
        }
    }
  };

  {
    // one step: wait for its DMA (STAGES - 2 later batches stay in flight), issue the DMA
    // STAGES - 1 steps ahead into the slot read last step, multiply, and finish the tile on
    // its last step
    auto step = [&](auto slot_c, int j) __attribute__((always_inline)) {
      constexpr int SL = decltype(slot_c)::value;
      const uint8_t* As = SL == 0 ? slot0 : (SL == 1 ? slot1 : slot2);
      int kt, tks;  // K step within the tile, the tile's K steps
      if constexpr (kRag) {
        kt = c_kt;
        tks = c_ks;
      } else {
        kt = j % ksteps;
        tks = ksteps;
      }
      if (kRoundSync && kt == 0 && j > 0) {  // a new round: arrive for the last one, wait for the XCD
        if (tid == 0) {
          const int q = j / ksteps;
          __hip_atomic_fetch_add(&p.sync[xcd], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const unsigned int tgt = round_target(q);
#pragma unroll 1
          for (int it = 0; it < kSyncSpins; ++it) {
            if (__hip_atomic_load(&p.sync[xcd], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= tgt) break;
            __builtin_amdgcn_s_sleep(2);
          }
        }
      }
      MOE_WAIT_VM(L_STAGE * (STAGES - 2));
      MOE_BARRIER();
      // the DMA of step j + STAGES - 1 goes to the slot read last step; its instructions are
      // spread over this step's MFMAs
      constexpr auto dslot = std::integral_constant<int, (SL + STAGES - 1) % STAGES>();
      issue_prep(j + STAGES - 1);
      if constexpr (!FP8) dma_now = kt != tks - 1;

      if constexpr (!FP8) {
        const uint8_t* Bs = As + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8_t af[TM], bfr[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) af[i] = *(const bf16x8_t*)(As + (ks ? fa_hi : fa_lo) + i * 16 * 128);
#pragma unroll
          for (int jj = 0; jj < TN; ++jj) {
            const int ro = (SWIGLU && jj >= TN / 2 ? BN / 2 + (jj - TN / 2) * 16 : jj * 16) * 128;
            bfr[jj] = *(const bf16x8_t*)(Bs + (ks ? fb_hi : fb_lo) + ro);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) {
              acc[i][jj] = mfma_bf16(af[i], bfr[jj], acc[i][jj]);
              dma_in(dslot, (ks * TM + i) * TN + jj, 2 * TM * TN);
            }
        }
      } else if constexpr (E8) {
        i32x8 af[TM], bfr[TN];
        int sa[TM], sw0, sw1;
        e8_read(As, kt, tks, af, bfr, sa, sw0, sw1);
        e8_math(dslot, af, bfr, sa, sw0, sw1);
      } else {
        i32x8 af[TM], bfr[TN];
        float s0[TM], s1[TM];
        fp8_read(As, kt, tks, af, bfr, s0, s1);
        fp8_math(dslot, af, bfr, s0, s1);
      }
      issue_scales();

      if (kt == tks - 1) {
        if constexpr (SWIGLU && PRE) epi_preact(ct);
        float v[TM][TO][4];
        epi_values(v);
        if (OUT == OUT_FP8) {
          epi_reduce(v);
          MOE_BARRIER();
        }
        epi_store(v, ct);
        if (OUT == OUT_FP8) MOE_BARRIER();  // s_red is rewritten by the next tile
        if (j + 1 < total_steps) ct = tile_of(kRag ? c_q + 1 : (j + 1) / ksteps, cur_c);
        if constexpr (!FP8) {
#pragma unroll
          for (int k = 0; k < L_ISSUE; ++k) issue_one(dslot, k);
        }
      }
      if constexpr (kRag) {
        if (kt == tks - 1) {
          ++c_q;
          c_kt = 0;
          c_ks = group_ksteps(ct.g);
        } else {
          ++c_kt;
        }
      }
    };

    int j = 0;
    for (; j + STAGES <= total_steps; j += STAGES) {
      step(std::integral_constant<int, 0>(), j);
      step(std::integral_constant<int, 1>(), j + 1);
      if constexpr (STAGES > 2) step(std::integral_constant<int, 2 % STAGES>(), j + 2);
    }
    if (j < total_steps) step(std::integral_constant<int, 0>(), j);
    if constexpr (STAGES > 2)
      if (j + 1 < total_steps) step(std::integral_constant<int, 1>(), j + 1);
  }
  MOE_WAIT_VM(0);  // the clamped tail DMA must land before the workgroup retires
  leave();
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v >= 8)
      cus = v / 8 * 8;
    else
      cus = 256;
  }
  return cus;
}

constexpr size_t kLdsBytes = 160 * 1024;

// Static LDS of one kernel instantiation (queried once).
template <int BM, int BN, int WGM, int WGN, int STAGES, int FP8, bool SWIGLU, int OUT, bool PRE>
size_t static_lds() {
  static size_t bytes = 0;
  if (bytes == 0) {
    hipFuncAttributes attr;
    const void* fn = reinterpret_cast<const void*>(&grouped_gemm_kernel<BM, BN, WGM, WGN, STAGES, FP8, SWIGLU, OUT, PRE>);
    if (hipFuncGetAttributes(&attr, fn) == hipSuccess)
      bytes = attr.sharedSizeBytes;
    else
      bytes = kLdsBytes;  // unknown: treat as full, so callers take a smaller configuration
  }
  return bytes;
}

template <int BM, int BN, int WGM, int WGN, int STAGES, int FP8, bool SWIGLU, int OUT, bool PRE>
bool fits(const GemmArgs& a) {
  return static_lds<BM, BN, WGM, WGN, STAGES, FP8, SWIGLU, OUT, PRE>() + (size_t)(a.n_groups + 1) * 4 <= kLdsBytes;
}

template <int BM, int BN, int WGM, int WGN, int STAGES, int FP8, bool SWIGLU, int OUT, bool PRE>
void launch(GemmArgs a, int64_t m_total, hipStream_t stream) {
  a.n_tiles = a.out_cols / (SWIGLU ? BN / 2 : BN);
  const int64_t mtiles = (m_total + (int64_t)a.n_groups * (BM - 1)) / BM;
  const int64_t upper = mtiles * a.n_tiles;
  if (upper <= 0) return;
  const int cus = device_cus();
  const int64_t grid = upper < cus ? ((upper + 7) / 8) * 8 : cus;
  const size_t dyn = (size_t)(a.n_groups + 1) * 4;  // the tile prefix table
  grouped_gemm_kernel<BM, BN, WGM, WGN, STAGES, FP8, SWIGLU, OUT, PRE><<<(unsigned)grid, WGM * WGN * 64, dyn, stream>>>(a);
}

// Row-block height for bf16 groups of about mu rows (the group sizes live on the device, so
// the host uses the mean): the expected row tiles per group, with a group's rows taken as
// normal with standard deviation sqrt(mu) (routing counts), times the relative cost of a
// tile step -- 160-row steps move ~11% more LDS bytes than 128-row steps (196 vs 176 KB).
// At 128 +- 11 rows per expert (T = 4096) 128-row blocks need ~1.5 tiles per expert, 160-row
// blocks ~1.0.
bool prefer_tall_rows(int64_t m_total, int n_groups) {
  const double mu = (double)m_total / n_groups;
  if (mu < 96.0) return false;
  const double sd = sqrt(mu);
  double e128 = 0, e160 = 0;
  for (int k = -8; k <= 8; ++k) {
    const double z = k * 0.375, w = exp(-0.5 * z * z), rows = fmax(1.0, mu + z * sd);
    e128 += w * ceil(rows / 128.0);
    e160 += w * ceil(rows / 160.0);
  }
  return e160 * 1.11 < e128;
}

// bf16: 8 waves of 64x64 (or 80x64 with 160-row blocks, see above), three-slot ring.
// E4M3: 8 waves of 64x64 and a three-slot ring
// where its LDS (147 KB of ring, the scale chunks and the tile table) fits, else two slots.
// Decode-sized groups: 64-row blocks, 8 waves of 64x32.
// Narrow bf16 outputs (N/2 or N not a multiple of 128 / 256): 128-column blocks, 4 waves.
template <int FP8, bool SWIGLU, int OUT, bool PRE>
void dispatch_as(const GemmArgs& a, int64_t m_total, bool small, bool narrow, hipStream_t stream) {
  if constexpr (!FP8) {
    if (narrow) {
      launch<64, 128, 1, 4, 3, FP8, SWIGLU, OUT, PRE>(a, m_total, stream);
      return;
    }
  }
  if (small) launch<64, 256, 1, 8, 3, FP8, SWIGLU, OUT, PRE>(a, m_total, stream);
  else if constexpr (!FP8) {
    if (prefer_tall_rows(m_total, a.n_groups) && fits<160, 256, 2, 4, 3, FP8, SWIGLU, OUT, PRE>(a))
      launch<160, 256, 2, 4, 3, FP8, SWIGLU, OUT, PRE>(a, m_total, stream);
    else
      launch<128, 256, 2, 4, 3, FP8, SWIGLU, OUT, PRE>(a, m_total, stream);
  } else {
    if (fits<128, 256, 2, 4, 3, FP8, SWIGLU, OUT, PRE>(a)) launch<128, 256, 2, 4, 3, FP8, SWIGLU, OUT, PRE>(a, m_total, stream);
    else launch<128, 256, 2, 4, 2, FP8, SWIGLU, OUT, PRE>(a, m_total, stream);
  }
}

// the preact kernels exist for the SwiGLU launches of bf16 and f32-scale E4M3 inputs
template <int FP8, bool SWIGLU, int OUT>
void dispatch(const GemmArgs& a, int64_t m_total, bool small, bool narrow, hipStream_t stream) {
  if constexpr (SWIGLU && FP8 != 2) {
    if (a.out_pre) {
      dispatch_as<FP8, SWIGLU, OUT, true>(a, m_total, small, narrow, stream);
      return;
    }
  }
  dispatch_as<FP8, SWIGLU, OUT, false>(a, m_total, small, narrow, stream);
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_grouped_gemm_workspace_size(void) { return moe::kGemmWsBytes; }

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
  MOE_REQUIRE(d->n_groups >= 1 && d->n_groups <= kMaxGroups && d->first_group >= 0, MOE_ERR_SHAPE,
              "moe_grouped_gemm: n_groups=%d first_group=%d", d->n_groups, d->first_group);
  MOE_REQUIRE(d->m_total >= 0 && d->m_total < ((int64_t)1 << 31), MOE_ERR_SHAPE, "moe_grouped_gemm: m_total=%lld",
              (long long)d->m_total);
  const int kstep_elems = fp8 ? 128 : 64;
  MOE_REQUIRE(d->K >= kstep_elems && d->K % kstep_elems == 0, MOE_ERR_SHAPE,
              "moe_grouped_gemm: K=%d must be a positive multiple of %d", d->K, kstep_elems);
  // column blocks: bf16 128 (SwiGLU: 64 + 64), E4M3 256 (SwiGLU: 128 + 128, one 1x128 h tile)
  const int ncols_min = fp8 ? 256 : 128;
  MOE_REQUIRE(d->N >= ncols_min && d->N % ncols_min == 0, MOE_ERR_SHAPE,
              "moe_grouped_gemm: N=%d must be a positive multiple of %d%s", d->N, ncols_min,
              swiglu ? " (N/2 gate + N/2 up rows)" : "");
  if (fp8) MOE_REQUIRE(d->a_scale && d->w_scale, MOE_ERR_NULL, "moe_grouped_gemm: FP8 inputs need a_scale and w_scale");
  MOE_REQUIRE(d->scale_fmt == MOE_SCALE_F32 || d->scale_fmt == MOE_SCALE_E8M0, MOE_ERR_DTYPE,
              "moe_grouped_gemm: unknown scale_fmt %d", d->scale_fmt);
  const bool e8 = fp8 && d->scale_fmt == MOE_SCALE_E8M0;
  MOE_REQUIRE(!e8 || d->K % 512 == 0, MOE_ERR_SHAPE,
              "moe_grouped_gemm: E8M0 scales need K a multiple of 512 (K=%d)", d->K);
  if (d->out_dtype == MOE_FP8_E4M3) MOE_REQUIRE(d->out_scale, MOE_ERR_NULL, "moe_grouped_gemm: FP8 output needs out_scale");
  MOE_REQUIRE(d->ws && d->ws_bytes >= kGemmWsBytes && aligned16(d->ws), MOE_ERR_WORKSPACE,
              "moe_grouped_gemm: workspace %zu < %zu bytes (or NULL / unaligned)", d->ws_bytes, kGemmWsBytes);
  const int esz = fp8 ? 1 : 2;
  const int osz = d->out_dtype == MOE_F32 ? 4 : (d->out_dtype == MOE_BF16 ? 2 : 1);
  const int out_cols = swiglu ? d->N / 2 : d->N;
  MOE_REQUIRE(d->lda >= d->K && (d->lda * esz) % 16 == 0, MOE_ERR_ALIGN, "moe_grouped_gemm: lda=%lld", (long long)d->lda);
  MOE_REQUIRE(d->ldo >= out_cols && (d->ldo * osz) % 16 == 0, MOE_ERR_ALIGN, "moe_grouped_gemm: ldo=%lld", (long long)d->ldo);
  MOE_REQUIRE(aligned16(d->a) && aligned16(d->w) && aligned16(d->out), MOE_ERR_ALIGN,
              "moe_grouped_gemm: a, w and out must be 16-byte aligned");
  MOE_REQUIRE(!fp8 || ((reinterpret_cast<uintptr_t>(d->a_scale) & 3u) == 0 && (reinterpret_cast<uintptr_t>(d->w_scale) & 3u) == 0),
              MOE_ERR_ALIGN, "moe_grouped_gemm: scales must be 4-byte aligned");
  const int64_t ldw = d->ldw ? d->ldw : d->K;
  MOE_REQUIRE(ldw >= d->K && (ldw * esz) % 16 == 0, MOE_ERR_ALIGN, "moe_grouped_gemm: ldw=%lld", (long long)d->ldw);
  MOE_REQUIRE((int64_t)d->N * ldw * esz < ((int64_t)1 << 31), MOE_ERR_SHAPE, "moe_grouped_gemm: one W[g] exceeds 2 GiB");
  MOE_REQUIRE(d->tail_groups >= 0 && d->tail_groups <= d->n_groups, MOE_ERR_SHAPE,
              "moe_grouped_gemm: tail_groups=%d must be in [0, n_groups=%d]", d->tail_groups, d->n_groups);
  if (d->tail_groups > 0) {
    MOE_REQUIRE(!swiglu && d->out_dtype == MOE_BF16, MOE_ERR_DTYPE,
                "moe_grouped_gemm: a split output needs epilogue NONE and a bf16 main output");
    MOE_REQUIRE(d->m_total == 0 || d->out_tail, MOE_ERR_NULL, "moe_grouped_gemm: out_tail is NULL");
    MOE_REQUIRE(d->ldo_tail >= out_cols && (d->ldo_tail * 4) % 16 == 0 && aligned16(d->out_tail), MOE_ERR_ALIGN,
                "moe_grouped_gemm: out_tail must be 16-byte aligned with ldo_tail >= %d (ldo_tail=%lld)", out_cols,
                (long long)d->ldo_tail);
  }

  MOE_REQUIRE(!d->k_offsets || (d->out_dtype == MOE_F32 && !swiglu && !e8), MOE_ERR_DTYPE,
              "moe_grouped_gemm: k_offsets needs an f32 output, epilogue NONE and f32 scales");
  if (d->out_preact) {
    MOE_REQUIRE(swiglu && !e8, MOE_ERR_DTYPE, "moe_grouped_gemm: out_preact needs the SwiGLU epilogue (bf16 or f32-scale FP8)");
    MOE_REQUIRE(aligned16(d->out_preact) && d->ldo_preact >= d->N && (d->ldo_preact * 4) % 16 == 0, MOE_ERR_ALIGN,
                "moe_grouped_gemm: out_preact must be 16-byte aligned with ldo_preact >= N (ldo_preact=%lld)",
                (long long)d->ldo_preact);
  }

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
  a.w_row_b = ldw * esz;
  a.out = static_cast<uint8_t*>(d->out);
  a.ldo_b = d->ldo * osz;
  a.out_scale = d->out_scale;
  a.out_scale_ld = out_cols / 128;
  a.tail_first = d->n_groups - d->tail_groups;
  a.out_tail = static_cast<uint8_t*>(d->out_tail);
  a.ldo_tail_b = d->ldo_tail * 4;
  a.out_cols = out_cols;
  a.n_tiles = 0;  // set per tile shape at launch
  a.sync = static_cast<unsigned int*>(d->ws);
  a.k_offs = d->k_offsets ? d->k_offsets + d->first_group : nullptr;
  a.out_pre = static_cast<uint8_t*>(d->out_preact);
  a.ldo_pre_b = d->ldo_preact * 4;
  const bool narrow = !fp8 && d->N % 256 != 0;

  // Tile shape by regime: many rows per expert -> 128-row blocks; few (decode) -> 64.
  const bool small = d->m_total / d->n_groups < 64;
  if (!fp8) {
    if (swiglu) dispatch<0, true, OUT_BF16>(a, d->m_total, small, narrow, stream);
    else if (d->out_dtype == MOE_BF16) dispatch<0, false, OUT_BF16>(a, d->m_total, small, narrow, stream);
    else dispatch<0, false, OUT_F32>(a, d->m_total, small, narrow, stream);
  } else if (!e8) {
    if (swiglu) {
      if (d->out_dtype == MOE_FP8_E4M3) dispatch<1, true, OUT_FP8>(a, d->m_total, small, narrow, stream);
      else dispatch<1, true, OUT_BF16>(a, d->m_total, small, narrow, stream);
    } else if (d->out_dtype == MOE_BF16) dispatch<1, false, OUT_BF16>(a, d->m_total, small, narrow, stream);
    else dispatch<1, false, OUT_F32>(a, d->m_total, small, narrow, stream);
  } else {
    if (swiglu) {
      if (d->out_dtype == MOE_FP8_E4M3) dispatch<2, true, OUT_FP8>(a, d->m_total, small, narrow, stream);
      else dispatch<2, true, OUT_BF16>(a, d->m_total, small, narrow, stream);
    } else if (d->out_dtype == MOE_BF16) dispatch<2, false, OUT_BF16>(a, d->m_total, small, narrow, stream);
    else dispatch<2, false, OUT_F32>(a, d->m_total, small, narrow, stream);
  }
  return check_launch("moe_grouped_gemm");
}
