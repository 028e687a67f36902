// Grouped expert FFN: two grouped GEMMs over the expert-sorted rows with the
// bias and activation fused into the epilogue of the first (GELU / ReLU /
// SwiGLU) and the bias into the second.
//
// Expert FFN: MoE Training: Mixture of Experts, "Basic MoE Architecture"
// (Linear(h, 4h), GELU, Linear(4h, h)); moe_code.py, class Expert (ReLU,
// biases; dropout is the identity in a forward pass); Moe survey, Mixtral
// count (three matrices per expert: a gated FFN, here SwiGLU).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on 128x128x64 block tiles, four waves
// of 64x64, operands staged through LDS with a 16-byte XOR swizzle (row & 7)
// so the 32 rows a fragment read touches fall in distinct banks, and double
// buffered with one barrier per K step. float32 path (float32 layers): a
// plain FMA kernel over the same tile map.
#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace moe {

// EPI_DGELU / EPI_DRELU (backward): C = acc * act'(z) with z read from Zin, the
// saved pre-activation laid out like C.
enum { EPI_GELU = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_NONE = 3, EPI_PARTIAL = 4, EPI_DGELU = 5,
       EPI_DRELU = 6 };

template <int EPI>
__device__ __forceinline__ float epilogue(float z1, float z3) {
  if (EPI == EPI_GELU) return gelu_erf(z1);
  if (EPI == EPI_RELU) return fmaxf(z1, 0.f);
  if (EPI == EPI_SWIGLU) return silu(z1) * z3;
  return z1;
}

// Locates M tile `mt` of the grouped row space. Group g owns rows
// [offsets[g], offsets[g+1]) (clamped to [0, rows_max], so malformed offsets
// can never address outside the row buffers), split into ceil(rows / BM)
// tiles in group order. Every wave of the block computes the same answer
// (lane l scans groups 5l .. 5l+4, then a wave prefix sum over lanes).
// Returns false when mt is past the last tile.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int G, int rows_max,
                                          int BM, int mt, int& g_out, int& row0_out,
                                          int& nrows_out) {
  constexpr int PER = 5;  // 64 lanes x 5 >= MOE_MAX_EXPERTS + 1 groups
  const int lane = threadIdx.x & 63;
  const int g0 = lane * PER;
  int o[PER + 1];
#pragma unroll
  for (int i = 0; i <= PER; ++i) {
    const int gi = g0 + i;
    o[i] = !offsets ? (gi == 0 ? 0 : rows_max)
                    : gi <= G ? min(max(offsets[gi], 0), rows_max) : rows_max;
  }
  int n[PER];
  int s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int gi = g0 + i;
    n[i] = (gi < G && o[i + 1] > o[i]) ? (o[i + 1] - o[i] + BM - 1) / BM : 0;
    s += n[i];
  }
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  const int total = __shfl(incl, 63, 64);
  if (mt >= total) return false;
  const int excl = incl - s;
  const bool mine = mt >= excl && mt < incl;
  const int owner = __ffsll((unsigned long long)__ballot(mine)) - 1;
  int g = 0, row0 = 0, nrows = 0;
  if (mine) {
    int acc = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (g == 0 && nrows == 0 && mt < acc + n[i]) {
        g = g0 + i;
        row0 = o[i] + (mt - acc) * BM;
        nrows = min(BM, o[i + 1] - row0);
      }
      acc += n[i];
    }
  }
  g_out = __shfl(g, owner, 64);
  row0_out = __shfl(row0, owner, 64);
  nrows_out = __shfl(nrows, owner, 64);
  return true;
}

// Per-wave view of the grouped row space (offsets null: one group of
// rows_max rows): lane l holds groups 5l .. 5l+4
// (first covered row, end row, tile count) and the exclusive prefix of tiles
// before its first group. `part` selects the rows covered: 0 all rows of
// every group in BM-row tiles; 1 the first floor(n / BM) BM-row tiles of each
// group of n rows; 2 the rows that part 1 leaves over (fewer than `big`), in
// BM-row tiles. Groups of at most skip_rows rows are left out (the streaming
// GEMM runs them); for the last group (g = G - 1) the bound is skip_last.
struct TileSpace {
  int s[5], e[5], n[5];
  int excl, incl, total;
};

__device__ __forceinline__ void tile_space_init(TileSpace& ts, const int32_t* __restrict__ offsets,
                                                int G, int rows_max, int BM, int part = 0,
                                                int big = 256, int skip_rows = 0,
                                                int skip_last = 0) {
  constexpr int PER = 5;
  const int lane = threadIdx.x & 63;
  const int g0 = lane * PER;
  int o[PER + 1];
#pragma unroll
  for (int i = 0; i <= PER; ++i) {
    const int gi = g0 + i;
    o[i] = !offsets ? (gi == 0 ? 0 : rows_max)
                    : gi <= G ? min(max(offsets[gi], 0), rows_max) : rows_max;
  }
  int sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int gi = g0 + i;
    const int rows0 = (gi < G && o[i + 1] > o[i]) ? o[i + 1] - o[i] : 0;
    // (groups the streaming GEMM takes)
    const int rows = rows0 > (gi == G - 1 ? skip_last : skip_rows) ? rows0 : 0;
    const int full = part == 0 ? 0 : rows / big * big;
    ts.s[i] = o[i] + (part == 2 ? full : 0);
    ts.e[i] = part == 1 ? o[i] + full : o[i] + rows;
    ts.n[i] = (ts.e[i] - ts.s[i] + BM - 1) / BM;
    sum += ts.n[i];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  ts.incl = incl;
  ts.excl = incl - sum;
  ts.total = __shfl(incl, 63, 64);
}

// Group, first row and row count of M tile mt (< ts.total); uniform over the wave.
__device__ __forceinline__ void tile_lookup(const TileSpace& ts, int mt, int BM, int& g_out,
                                            int& row0_out, int& nrows_out) {
  constexpr int PER = 5;
  const int lane = threadIdx.x & 63;
  const bool mine = mt >= ts.excl && mt < ts.incl;
  const int owner = __ffsll((unsigned long long)__ballot(mine)) - 1;
  int g = -1, row0 = 0, nrows = 0;
  if (mine) {
    int acc = ts.excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (g < 0 && mt < acc + ts.n[i]) {
        g = lane * PER + i;
        row0 = ts.s[i] + (mt - acc) * BM;
        nrows = min(BM, ts.e[i] - row0);
      }
      acc += ts.n[i];
    }
  }
  g_out = __shfl(g, owner, 64);
  row0_out = __shfl(row0, owner, 64);
  nrows_out = __shfl(nrows, owner, 64);
}

__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

template <int EPI>
__device__ __forceinline__ float epilogue_bf16(float z1, float z3) {
  if (EPI == EPI_GELU) return gelu_poly(z1);
  if (EPI == EPI_RELU) return fmaxf(z1, 0.f);
  if (EPI == EPI_SWIGLU) return silu_fast(z1) * z3;
  if (EPI == EPI_DGELU) return z1 * gelu_grad_poly(z3);
  if (EPI == EPI_DRELU) return z3 > 0.f ? z1 : 0.f;
  return z1;
}

// One 8-element K fragment of v_mfma_f32_32x32x16_bf16 read transposed out of
// a row-major LDS tile: two ds_read_b64_tr_b16, the second 4 rows after the
// first (lane layout: gemm_bf16_kernel's KMB note).
// PITCH: bytes per LDS row.
template <int PITCH = 256>
__device__ __forceinline__ bf16x8 lds_tr_frag(const u32x4* smem, uint32_t byte) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  lds_s16x4* p = (lds_s16x4*)((__attribute__((address_space(3))) char*)smem + byte);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p + PITCH / 2);
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Grouped GEMM, C[r, n] = epi(sum_k A[r, k] W_g[n, k] + b_g[n]); group g < E
// takes expert weights W + g N K, group E (shared expert) takes Ws.
//
// One 128 x 128 output tile per block (SwiGLU: 128 x 64 of W1 and of W3 side by
// side), K step 64, four waves as 2 x 2, each wave 64 x 64 (SwiGLU 64 x 32 per
// operand) on v_mfma_f32_32x32x16_bf16 with 64 float32 accumulators per lane.
// 64 KB of LDS and at most 256 registers per lane let two blocks share a CU,
// so one block's load waits and epilogue overlap the other's MFMAs. Operands
// move global -> registers -> LDS with a two-step register prefetch: the loads
// of K step k + 2 are issued while step k is multiplied, and the registers of
// step k + 1 go to the other LDS stage at the end of step k. A stage holds 256
// rows of 128 bytes (128 A rows, then the B rows); 16-byte chunk c of row r
// sits at chunk c ^ ((r >> 1) & 7), so the 16 lanes of one LDS cycle (16
// consecutive rows, one chunk) cover all 64 banks once. Within a K step the
// fragments of sub-step s + 1 are read while sub-step s multiplies. The MFMA
// takes the weight fragment first, so a lane's accumulators hold four
// consecutive output columns of one row. The epilogue adds the bias, applies
// the activation, stages the bf16 tile in LDS and writes whole 256-byte row
// segments. Blocks are dispatched to the 8 XCDs round-robin; the block id is
// remapped so that each XCD runs a contiguous range of tiles, ordered in
// groups of 8 M tiles, whose operands then meet in that XCD's L2.
//
// KMB (backward dZ and dX GEMMs): the weights are read as stored, K-major,
//   C[r, n] = epi(sum_k A[r, k] W_g[k, n]),
// W_g [K][N] at W + g ksplit N for K steps below ksplit and W3_g at
// W3 + g ksplit N for the rest (SwiGLU's dX, K = 2F over [W1; W3]; ksplit = K
// otherwise); the shared expert takes Ws / Ws3. The B part of a stage then
// holds 64 K rows of 256 bytes (128 columns), 16-byte chunk c of row k at
// c ^ 4 (k & 3), and each B fragment is two ds_read_b64_tr_b16: in each group
// of 16 lanes, lane 4a + b receives element b of the 8-byte pieces addressed
// by lanes a, a + 4, a + 8 and a + 12, so lane x addresses row x / 4 (of four
// consecutive K rows) and columns 4 (x % 4) .. + 3 to receive four consecutive
// K values of column x. The four rows of a 32-lane half land in four distinct
// 64-byte bank groups.
template <int EPI, bool HAS_BIAS, bool KMB = false>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* __restrict__ W3,
    const float* __restrict__ bias, const bf16* __restrict__ Ws, const bf16* __restrict__ Ws3,
    const float* __restrict__ bias_s, int E, int G, const int32_t* __restrict__ offsets,
    int rows_max, void* __restrict__ Cv, int N, int K, int part, const int32_t* __restrict__ arows,
    int kparts, const bf16* __restrict__ Zin, int skip_rows, int skip_last, int ksplit,
    float* __restrict__ colsum, int aux_tiles) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  static_assert(!KMB || !GATED, "K-major weights: ungated backward GEMMs");
  constexpr bool DACT = EPI == EPI_DGELU || EPI == EPI_DRELU;
  constexpr int BM = 128, BK = 64, CH = BK / 8;   // 8 chunks of 16 B per LDS row
  constexpr int NB = GATED ? 2 : 1;
  constexpr int BN = GATED ? 64 : 128;            // columns per B operand
  constexpr int WN = BN / 2;                       // per wave, per operand
  constexpr int TM = 2, TN = WN / 32;
  constexpr int ROWS = BM + NB * BN;               // 256 LDS rows per stage
  constexpr int STAGE = ROWS * CH;                 // u32x4 per stage (32 KB)
  constexpr int GROUP_M = 8;
  constexpr int CQ = BN / 8;                       // 16-byte chunks per output row
  __shared__ u32x4 smem[2 * STAGE];
  bf16* __restrict__ C = reinterpret_cast<bf16*>(Cv);

  TileSpace ts;
  tile_space_init(ts, offsets, G, rows_max, BM, part, kGemmBigBM, skip_rows, skip_last);
  const int mtiles = __builtin_amdgcn_readfirstlane(ts.total);
  const int ntn = N / BN;
  const int tiles = mtiles * ntn;
  // Persistent blocks: block b takes tiles b, b + P, b + 2P, ... of the
  // XCD-aware order (P = gridDim.x, a multiple of 8, so a block stays on its
  // XCD's contiguous range of tiles).
  // With kparts > 1 (EPI_PARTIAL only) each tile's K steps are cut into kparts
  // equal ranges, one work item each, whose float32 sums go to plane
  // (item % kparts) of C; a separate pass adds the planes.
  const int P = gridDim.x;
  const int nk = K / BK;
  const int len = nk / kparts;   // >= 4 and even (host's choice of kparts)
  const int items = tiles * kparts;
  int it = blockIdx.x;
  if (it >= items) return;
  const int t8 = tiles & ~7;
  const int per_group = GROUP_M * ntn;
  int g, row0, nrows, n0, mtile;
  const bf16* Wg;
  const bf16* W3g;
  const float* bg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31;
  const int fk = lane >> 5;
  // Loads: thread t covers chunk t & 7 of tile rows (t >> 3) + 32 i, i = 0..3,
  // of A and of B; all of them share (row >> 1) & 7 = (t >> 4) & 7.
  const int lr = tid >> 3;
  const int lc = tid & 7;
  const int wslot = lr * CH + (lc ^ ((tid >> 4) & 7));
  const int rsw = (fr >> 1) & 7;                   // fragment rows: (r >> 1) & 7

  // Uniform base addresses and per-thread 32-bit byte offsets (A rows past the
  // tile's end repeat its last row). W3 rows of the B part start at LDS row
  // BN (= 64) for SwiGLU.
  // A row r of the tile is row row0 + r of A, or, with arows, row arows[row0 + r]
  // (the expert-sorted gather of token rows, fused here).
  const char* b_s;
  const char* b3_s;
  const char* ar0;
  const char* ar1;
  const char* ar2;
  const char* ar3;
  int kp, kbase;   // K range of the current work item and its first K step
  // work item itx: tile itx / kparts of the XCD-aware order (group, rows,
  // columns, operand addresses) and K range itx % kparts
  auto setup = [&](int itx) {
    const int ti = itx / kparts;
    kp = itx - ti * kparts;
    kbase = kp * len;
    const int t = ti < t8 ? (ti & 7) * (t8 >> 3) + (ti >> 3) : ti;
    const int grp = t / per_group;
    const int first_m = grp * GROUP_M;
    const int in = t - grp * per_group;
    const int gm = min(mtiles - first_m, GROUP_M);
    const int mt = first_m + in % gm;
    const int nt = in / gm;
    mtile = mt;
    tile_lookup(ts, mt, BM, g, row0, nrows);
    // uniform over the block: keep them in scalar registers
    g = __builtin_amdgcn_readfirstlane(g);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    n0 = nt * BN;
    if constexpr (KMB) {
      Wg = g < E ? W + (int64_t)g * ksplit * N : Ws;
      W3g = g < E ? (W3 ? W3 + (int64_t)g * ksplit * N : nullptr) : Ws3;
      bg = HAS_BIAS ? (g < E ? bias + (int64_t)g * N : bias_s) : nullptr;
      b_s = reinterpret_cast<const char*>(Wg + n0);
      b3_s = W3g ? reinterpret_cast<const char*>(W3g + n0) : b_s;
    } else {
      Wg = g < E ? W + (int64_t)g * N * K : Ws;
      W3g = GATED ? (g < E ? W3 + (int64_t)g * N * K : Ws3) : Wg;
      bg = HAS_BIAS ? (g < E ? bias + (int64_t)g * N : bias_s) : nullptr;
      b_s = reinterpret_cast<const char*>(Wg + (int64_t)n0 * K);
      b3_s = GATED ? reinterpret_cast<const char*>(W3g + (int64_t)(n0 - BN) * K) : b_s;
    }
    int rr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + min(lr + 32 * i, nrows - 1);
      rr[i] = arows ? arows[r] : r;
    }
    const bf16* a0 = A + lc * 8;
    ar0 = reinterpret_cast<const char*>(a0 + (int64_t)rr[0] * K);
    ar1 = reinterpret_cast<const char*>(a0 + (int64_t)rr[1] * K);
    ar2 = reinterpret_cast<const char*>(a0 + (int64_t)rr[2] * K);
    ar3 = reinterpret_cast<const char*>(a0 + (int64_t)rr[3] * K);
  };
  // B loads: K-major, thread t covers chunk t & 15 of K rows (t >> 4) + 16 i
  // (byte offsets within one K step's 64 rows); else chunk t & 7 of rows
  // (t >> 3) + 32 i of the [N][K] tile
  const uint32_t bo0 = KMB ? (uint32_t)((tid >> 4) * N + (tid & 15) * 8) * 2u
                           : (uint32_t)(lr * K + lc * 8) * 2u;
  const uint32_t bstep = KMB ? (uint32_t)(32 * N) : (uint32_t)(64 * K);   // 16 / 32 rows
  const uint32_t bo1 = bo0 + bstep;
  const uint32_t bo2 = bo0 + 2 * bstep;
  const uint32_t bo3 = bo0 + 3 * bstep;
  const int wslot_b = BM * CH + (tid >> 4) * 16 + ((tid & 15) ^ (((tid >> 4) & 3) << 2));

  // LDS fragment rows: f = 0, 1 are A sub-tiles i = f; f = 2, 3 are B sub-tiles
  // jb = f - 2 (column block j of W, or W1 / W3 for SwiGLU).
  static_assert(TM == 2 && NB * TN == 2, "fragment plan");
  int fbase[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int jb = f - 2;
    const int row = f < 2 ? wm * 64 + f * 32 + fr
                          : BM + (NB == 1 ? wn * WN + jb * 32 : jb * BN + wn * WN) + fr;
    fbase[f] = row * CH;
  }
  constexpr int kRO[4] = {0, 2, 1, 3};   // fragment read order
  int cidx[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) cidx[s4] = (s4 * 2 + fk) ^ rsw;
  // K-major B fragments (jb = 0, 1): byte offset in the stage of the lane's
  // first transposed read (K rows 8 (lane / 32) + (lane % 16) / 4 of the
  // sub-step; the second read is 4 rows on)
  uint32_t toff[2];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int x = lane & 15, hq = (lane >> 4) & 1;
    const int krow = 8 * fk + (x >> 2);
    const int chunk = (wn * WN + jb * 32) / 8 + 2 * hq + ((x & 3) >> 1);
    toff[jb] = (uint32_t)((BM * CH + krow * 16 + (chunk ^ ((krow & 3) << 2))) * 16 + (x & 1) * 8);
  }

  // register stages for even / odd K steps (named registers, not arrays, so
  // that they stay in VGPRs)
  struct Regs { u32x4 v0, v1, v2, v3, v4, v5, v6, v7; };
  Regs r0, r1;
  bf16x8 fr0[4], fr1[4];   // fragments of two consecutive sub-steps
  f32x16 acc[4];           // acc[i + 2 jb] = A sub-tile i times B sub-tile jb

#define MOE_SB() __builtin_amdgcn_sched_barrier(0)
#define MOE_G(R, kt, i)                                                              \
  do {                                                                               \
    const uint32_t kb_ = (uint32_t)(kbase + (kt)) * (BK * 2);                        \
    if ((i) == 0) R.v0 = *reinterpret_cast<const u32x4*>(ar0 + kb_);                 \
    if ((i) == 1) R.v1 = *reinterpret_cast<const u32x4*>(ar1 + kb_);                 \
    if ((i) == 2) R.v2 = *reinterpret_cast<const u32x4*>(ar2 + kb_);                 \
    if ((i) == 3) R.v3 = *reinterpret_cast<const u32x4*>(ar3 + kb_);                 \
    if constexpr (KMB) {                                                             \
      const int kg_ = (kbase + (kt)) * BK;                                           \
      const char* bk_ = kg_ < ksplit ? b_s + (int64_t)kg_ * N * 2                    \
                                     : b3_s + (int64_t)(kg_ - ksplit) * N * 2;       \
      if ((i) == 4) R.v4 = *reinterpret_cast<const u32x4*>(bk_ + bo0);               \
      if ((i) == 5) R.v5 = *reinterpret_cast<const u32x4*>(bk_ + bo1);               \
      if ((i) == 6) R.v6 = *reinterpret_cast<const u32x4*>(bk_ + bo2);               \
      if ((i) == 7) R.v7 = *reinterpret_cast<const u32x4*>(bk_ + bo3);               \
    } else {                                                                         \
      if ((i) == 4) R.v4 = *reinterpret_cast<const u32x4*>(b_s + kb_ + bo0);         \
      if ((i) == 5) R.v5 = *reinterpret_cast<const u32x4*>(b_s + kb_ + bo1);         \
      if ((i) == 6) R.v6 = *reinterpret_cast<const u32x4*>(b3_s + kb_ + bo2);        \
      if ((i) == 7) R.v7 = *reinterpret_cast<const u32x4*>(b3_s + kb_ + bo3);        \
    }                                                                                \
  } while (0)
#define MOE_W(R, st, i)                                                              \
  do {                                                                               \
    u32x4* d_ = smem + (st) * STAGE + wslot;                                         \
    u32x4* db_ = smem + (st) * STAGE + wslot_b;                                      \
    if ((i) == 0) d_[0] = R.v0;                                                      \
    if ((i) == 1) d_[32 * CH] = R.v1;                                                \
    if ((i) == 2) d_[64 * CH] = R.v2;                                                \
    if ((i) == 3) d_[96 * CH] = R.v3;                                                \
    if constexpr (KMB) {                                                             \
      if ((i) == 4) db_[0] = R.v4;                                                   \
      if ((i) == 5) db_[16 * 16] = R.v5;                                             \
      if ((i) == 6) db_[32 * 16] = R.v6;                                             \
      if ((i) == 7) db_[48 * 16] = R.v7;                                             \
    } else {                                                                         \
      if ((i) == 4) d_[BM * CH] = R.v4;                                              \
      if ((i) == 5) d_[(BM + 32) * CH] = R.v5;                                       \
      if ((i) == 6) d_[(BM + 64) * CH] = R.v6;                                       \
      if ((i) == 7) d_[(BM + 96) * CH] = R.v7;                                       \
    }                                                                                \
  } while (0)
#define MOE_R(F, st, s4, f)                                                          \
  do {                                                                               \
    if (KMB && (f) >= 2)                                                             \
      F[f] = lds_tr_frag(smem, (uint32_t)((st) * STAGE * 16 + (s4) * 4096) + toff[(f) & 1]); \
    else                                                                             \
      F[f] = __builtin_bit_cast(bf16x8, smem[(st) * STAGE + fbase[f] + cidx[s4]]);   \
  } while (0)
#define MOE_M(F, q)                                                                  \
  acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[2 + ((q) >> 1)], F[(q) & 1], acc[q], 0, 0, 0)
  // One K step from LDS stage st: 16 MFMAs in four sub-steps, MFMA q taking
  // A sub-tile q & 1 and B sub-tile q >> 1; fragments are read in the order
  // A0 B0 A1 B1 so that each MFMA waits only for the reads it needs. Each MFMA
  // is followed by one fragment read of the next sub-step and, in sub-steps 0 / 1,
  // two global loads of register set RG (step KL) or, in sub-steps 2 / 3, one
  // LDS write of register set RW to the other stage. LD / WR switch those off.
#define MOE_STEP(st, RG, KL, LD, RW, WR)                                             \
  do {                                                                               \
    MOE_R(fr0, st, 0, 0); MOE_R(fr0, st, 0, 2); MOE_R(fr0, st, 0, 1);                \
    MOE_R(fr0, st, 0, 3); MOE_SB();                                                  \
    _Pragma("unroll") for (int k_ = 0; k_ < 4; ++k_) {                               \
      MOE_M(fr0, k_); MOE_SB(); MOE_R(fr1, st, 1, kRO[k_]); MOE_SB();                     \
      if (LD) { MOE_G(RG, KL, 2 * k_); MOE_G(RG, KL, 2 * k_ + 1); }                  \
      MOE_SB();                                                                      \
    }                                                                                \
    _Pragma("unroll") for (int k_ = 0; k_ < 4; ++k_) {                               \
      MOE_M(fr1, k_); MOE_SB(); MOE_R(fr0, st, 2, kRO[k_]); MOE_SB();                     \
    }                                                                                \
    _Pragma("unroll") for (int k_ = 0; k_ < 4; ++k_) {                               \
      MOE_M(fr0, k_); MOE_SB(); MOE_R(fr1, st, 3, kRO[k_]); MOE_SB();                     \
      if (WR) MOE_W(RW, 1 - (st), k_);                                               \
      MOE_SB();                                                                      \
    }                                                                                \
    _Pragma("unroll") for (int k_ = 0; k_ < 4; ++k_) {                               \
      MOE_M(fr1, k_); MOE_SB();                                                      \
      if (WR) MOE_W(RW, 1 - (st), 4 + k_);                                           \
      MOE_SB();                                                                      \
    }                                                                                \
  } while (0)

  // Steps kbase .. kbase + len - 1 (len >= 4 and even); the last two are
  // peeled so that the loop body has no branches.
  setup(it);
#pragma unroll
  for (int i = 0; i < 8; ++i) MOE_G(r0, 0, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) MOE_G(r1, 1, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) MOE_W(r0, 0, i);
  __syncthreads();
  for (;;) {
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k4][r] = 0.f;
  for (int kt = 0; kt < len - 2; kt += 2) {
    // even step kt: stage 0 holds it, r1 holds step kt + 1, r0 is loaded with kt + 2
    MOE_STEP(0, r0, kt + 2, true, r1, true);
    __syncthreads();
    // odd step kt + 1: stage 1 holds it, r0 holds step kt + 2, r1 is loaded with kt + 3
    MOE_STEP(1, r1, kt + 3, true, r0, true);
    __syncthreads();
  }
  MOE_STEP(0, r0, 0, false, r1, true);
  __syncthreads();
  MOE_STEP(1, r1, 0, false, r0, false);

  // The registers r0 / r1 are free now: the first two K steps of this block's
  // next tile are loaded into them before the epilogue of this one, so their
  // latency is spent under the epilogue instead of before the next K loop.
  const int cur_row0 = row0, cur_nrows = nrows, cur_n0 = n0, cur_kp = kp, cur_mt = mtile;
  const float* cur_bg = bg;
  const int itn = it + P;
  const bool more = itn < items;
  if (more) {
    setup(itn);
#pragma unroll
    for (int i = 0; i < 8; ++i) MOE_G(r0, 0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) MOE_G(r1, 1, i);
  }

  if constexpr (EPI == EPI_PARTIAL) {
    // float32 sums straight to plane cur_kp of C: [kparts][rows_max][N] by row,
    // or with aux_tiles > 0 [kparts][aux_tiles * 128][N] by M tile (row
    // 128 mt + m; tiles from aux_tiles on are not written: only malformed
    // offsets make that many). Lane (fr, fk) holds 4 consecutive columns of each
    // 8-column group.
    const int64_t prow = aux_tiles > 0 ? (int64_t)cur_mt * BM : cur_row0;
    const int64_t plane = aux_tiles > 0 ? (int64_t)aux_tiles * BM : rows_max;
    float* __restrict__ Cp = reinterpret_cast<float*>(Cv) + (int64_t)cur_kp * plane * N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = wm * 64 + i * 32 + fr;
      if (m < cur_nrows && (aux_tiles == 0 || cur_mt < aux_tiles)) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x4 v = {acc[i + 2 * j][qd * 4 + 0], acc[i + 2 * j][qd * 4 + 1],
                             acc[i + 2 * j][qd * 4 + 2], acc[i + 2 * j][qd * 4 + 3]};
            *reinterpret_cast<f32x4*>(Cp + (prow + m) * N + cur_n0 + wn * WN + j * 32 + qd * 8 +
                                      fk * 4) = v;
          }
      }
    }
  } else if constexpr (DACT) {
    // Backward epilogue C = acc * act'(z) (no bias): the float32 tile is staged
    // in LDS (64 KB: both operand stages), 16-byte chunk q (0..31) of row m at
    // q ^ (m & 31), so that 16 consecutive lanes of a write or a read hit 16
    // distinct chunks; then thread t takes 8 consecutive columns of rows
    // t / 16 + 16 p, reading z and writing dZ with whole 256-byte row segments.
    // The z loads are issued right after the staging writes (the accumulators
    // are free then), so that their latency is spent in the barrier. With
    // colsum, the tile's column sums of the rounded dZ (rows in order: each
    // thread's 8 rows, then the 16 row groups) go to colsum[mt][n] for M tile mt
    // of the tile space (the bias gradient adds a group's tiles in order).
    __syncthreads();   // every wave is done reading the operand stages
    f32x4* st4 = reinterpret_cast<f32x4*>(smem);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = wm * 64 + i * 32 + fr;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int q = wn * (WN / 4) + j * 8 + qd * 2 + fk;
          const f32x4 v = {acc[i + 2 * j][qd * 4 + 0], acc[i + 2 * j][qd * 4 + 1],
                           acc[i + 2 * j][qd * 4 + 2], acc[i + 2 * j][qd * 4 + 3]};
          st4[m * 32 + (q ^ (m & 31))] = v;
        }
    }
    u32x4 zq[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int m = (tid >> 4) + 16 * p;
      const u32x4 z0 = {0u, 0u, 0u, 0u};
      zq[p] = m < cur_nrows ? *reinterpret_cast<const u32x4*>(Zin + (int64_t)(cur_row0 + m) * N +
                                                                cur_n0 + (tid & 15) * 8)
                            : z0;
    }
    __syncthreads();
    float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int m = (tid >> 4) + 16 * p;
      const int c2 = (tid & 15) * 2;
      if (m < cur_nrows) {
        const f32x4 a = st4[m * 32 + (c2 ^ (m & 31))];
        const f32x4 b = st4[m * 32 + ((c2 + 1) ^ (m & 31))];
        const float dh[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        const uint32_t zw[4] = {zq[p].x, zq[p].y, zq[p].z, zq[p].w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = epilogue_bf16<EPI>(dh[2 * e], bf16_bits_to_f32(zw[e] & 0xffffu));
          const float hi = epilogue_bf16<EPI>(dh[2 * e + 1], bf16_bits_to_f32(zw[e] >> 16));
          o[e] = pack_bf16x2(lo, hi);
        }
        const u32x4 ov = {o[0], o[1], o[2], o[3]};
        *reinterpret_cast<u32x4*>(C + (int64_t)(cur_row0 + m) * N + cur_n0 + (tid & 15) * 8) = ov;
        if (colsum) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            cs[2 * e] += bf16_bits_to_f32(o[e] & 0xffffu);
            cs[2 * e + 1] += bf16_bits_to_f32(o[e] >> 16);
          }
        }
      }
    }
    if (colsum) {
      __syncthreads();   // the staged tile has been read
      float* red = reinterpret_cast<float*>(smem);   // [16 row groups][128 columns]
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(tid >> 4) * 128 + (tid & 15) * 8 + e] = cs[e];
      __syncthreads();
      if (tid < 128 && cur_mt < aux_tiles) {   // (tiles past the buffer: malformed offsets)
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) sum += red[q * 128 + tid];
        colsum[(int64_t)cur_mt * N + cur_n0 + tid] = sum;
      }
    }
  } else {
  // Epilogue. Register r of a 32x32 accumulator holds row (lane % 32) and
  // column 8 (r / 4) + 4 (lane / 32) + r % 4 of the sub-tile, so lane (fr, fk)
  // owns 8 bytes of 16-byte output chunk q = wn WN / 8 + 4 j + r / 4.
  float4 bv[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      bv[j][qd] = HAS_BIAS ? *reinterpret_cast<const float4*>(cur_bg + cur_n0 + wn * WN + j * 32 + qd * 8 + fk * 4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();   // every wave is done reading the operand stages
  // bf16 tile staged as BM rows of CQ chunks; chunk q of row m at q ^ swz(m)
  uint2* st8 = reinterpret_cast<uint2*>(smem);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * 64 + i * 32 + fr;
    const int swz = CQ == 16 ? (m & 15) : ((m >> 1) & 7);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float4 bq = bv[j][qd];
        const float z[4] = {acc[i + 2 * j][qd * 4 + 0] + bq.x, acc[i + 2 * j][qd * 4 + 1] + bq.y,
                            acc[i + 2 * j][qd * 4 + 2] + bq.z, acc[i + 2 * j][qd * 4 + 3] + bq.w};
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = epilogue_bf16<EPI>(z[e], GATED ? acc[i + 2][qd * 4 + e] : 0.f);
        uint2 u;
        u.x = pack_bf16x2(v[0], v[1]);
        u.y = pack_bf16x2(v[2], v[3]);
        const int q = wn * (WN / 8) + j * 4 + qd;
        st8[(m * CQ + (q ^ swz)) * 2 + fk] = u;
      }
    }
  }
  __syncthreads();
  // 16 (SwiGLU 8) consecutive threads write one row's contiguous segment
#pragma unroll
  for (int p = 0; p < BM * CQ / 256; ++p) {
    const int idx = p * 256 + tid;
    const int m = idx / CQ, q = idx % CQ;
    const int swz = CQ == 16 ? (m & 15) : ((m >> 1) & 7);
    if (m < cur_nrows)
      *reinterpret_cast<u32x4*>(C + (int64_t)(cur_row0 + m) * N + cur_n0 + q * 8) = smem[m * CQ + (q ^ swz)];
  }
  }
  if (!more) break;
  __syncthreads();   // the staged tile has been read out of stage 0
#pragma unroll
  for (int i = 0; i < 8; ++i) MOE_W(r0, 0, i);
  __syncthreads();
  it = itn;
  }
}

#undef MOE_SB
#undef MOE_G
#undef MOE_W
#undef MOE_R
#undef MOE_M
#undef MOE_STEP

// Weight gradient straight from the expert-sorted row buffers (backward pass):
// for group g,
//   C_g[m, n] = sum over rows r in [so[g], so[g + 1]) of A[r, m] B[r, n],
// A [rows][lda] and B [rows][ldb] bf16 row-major, C_g float32 [M][N] at
// C + g M N for a routed expert (g < E) and Cs for the shared expert (g == E).
// Both operands are K-major (K runs over rows), so a stage holds two tiles of
// 64 rows x 128 columns (A's, then B's), 16-byte chunk c of row k at
// c ^ 4 (k & 3), and every MFMA fragment is two ds_read_b64_tr_b16
// (lds_tr_frag; lane layout in gemm_bf16_kernel's KMB note). Rows past the
// group's end are loaded as zeros (buffer loads range-checked against the
// group's rows) and an empty group yields C_g = 0. 128 x 128 tile, four
// waves of 64 x 64, K step 64 with the next two steps in registers, one tile per
// block, the B fragment first in each MFMA so that a lane's accumulators hold
// four consecutive columns n; XCD-aware tile order (a group's tiles in groups of
// 8 M tiles on one XCD). Requires M, N multiples of 128 and lda, ldb < 2^24.
__global__ __launch_bounds__(256, 2) void gemm_wgrad_tn_kernel(
    const bf16* __restrict__ A, int lda, const bf16* __restrict__ B, int ldb,
    const int32_t* __restrict__ so, int G, int E, int M, int N, float* __restrict__ C,
    float* __restrict__ Cs) {
  constexpr int BM = 128, BN = 128, BK = 64, TC = 16;   // 16 chunks of 16 B per LDS row
  constexpr int HALF = BK * TC;                          // chunks of one operand tile
  constexpr int STAGE = 2 * HALF;                        // 32 KB
  constexpr int GROUP_M = 8;
  __shared__ u32x4 smem[2 * STAGE];
  const int mtn = M / BM, ntn = N / BN;
  const int ntb = wgrad_run(ntn);            // consecutive n tiles per block
  const int nrun = ntn / ntb, per = mtn * nrun;
  const int tiles = G * per;
  const int b = blockIdx.x;
  if (b >= tiles) return;
  const int t8 = tiles & ~7;
  const int t = b < t8 ? (b & 7) * (t8 >> 3) + (b >> 3) : b;
  const int g = t / per;
  const int in = t - g * per;
  const int grp = in / (GROUP_M * nrun);
  const int first_m = grp * GROUP_M;
  const int gm = min(mtn - first_m, GROUP_M);
  const int in2 = in - grp * GROUP_M * nrun;
  const int m0 = (first_m + in2 % gm) * BM;
  int n0 = (in2 / gm) * ntb * BN;
  // uniform over the block: scalar registers (the buffer descriptors below
  // must be scalar)
  const int r0 = __builtin_amdgcn_readfirstlane(so[g]);
  const int nr = __builtin_amdgcn_readfirstlane(so[g + 1]) - r0;   // the group's rows
  int len = (nr + BK - 1) / BK;   // K steps, made even and at least 2
  len = len < 2 ? 2 : (len + 1) & ~1;
  const int tid = threadIdx.x;
  if (nr <= 0) {
    // a group without rows (an expert that received no token): its gradient
    // is zero; the tile is stored straight away, in the row segments of the
    // epilogue below, with no operand loads
    float* __restrict__ Cz = (g < E ? C + (int64_t)g * M * N : Cs) + (int64_t)m0 * N + n0 +
                             (tid & 31) * 4;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < ntb; ++it)
#pragma unroll
      for (int p = 0; p < 16; ++p)
        __builtin_nontemporal_store(zero, reinterpret_cast<f32x4*>(Cz + it * BN + (int64_t)(p * 8 + (tid >> 5)) * N));
    return;
  }
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31;
  const int fk = lane >> 5;
  // loads: thread t covers chunk t & 15 of rows (t >> 4) + 16 i, i = 0..3, of
  // both tiles
  const int lr = tid >> 4;
  const int lc = tid & 15;
  const int wslot = lr * TC + (lc ^ ((lr & 3) << 2));
  const uint32_t ao = (uint32_t)(lr * lda + m0 + lc * 8) * 2u;   // within a step's rows
  uint32_t bo = (uint32_t)(lr * ldb + n0 + lc * 8) * 2u;          // (+ 256 per n tile)
  const uint32_t astep = (uint32_t)(32 * lda), bstep = (uint32_t)(32 * ldb);   // 16 rows
  // fragment byte offsets in a stage (sub-tile j of the wave's A / B columns;
  // + 4096 per 16-row sub-step)
  uint32_t fa[2], fb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int x = lane & 15, hq = (lane >> 4) & 1;
    const int krow = 8 * fk + (x >> 2);
    const int sw = (krow & 3) << 2;
    const int ca = (wm * 64 + j * 32) / 8 + 2 * hq + ((x & 3) >> 1);
    const int cb = (wn * 64 + j * 32) / 8 + 2 * hq + ((x & 3) >> 1);
    fa[j] = (uint32_t)((krow * TC + (ca ^ sw)) * 16 + (x & 1) * 8);
    fb[j] = (uint32_t)((HALF + krow * TC + (cb ^ sw)) * 16 + (x & 1) * 8);
  }
  constexpr int kRO[4] = {0, 2, 1, 3};   // fragment read order: A0 B0 A1 B1
  struct Regs { u32x4 v0, v1, v2, v3, v4, v5, v6, v7; };
  Regs r0v, r1v;
  bf16x8 fr0[4], fr1[4];   // [0], [1]: A sub-tiles; [2], [3]: B sub-tiles
  f32x16 acc[4];           // acc[i + 2 j] = B sub-tile j times A sub-tile i

#define WT_SB() __builtin_amdgcn_sched_barrier(0)
  // register set R <- K step kt: loads i = 0..3 from A, 4..7 from B, through
  // buffer descriptors that span only the step's rows inside the group, so the
  // rows past its end read as zeros (the hardware's range check; nothing past
  // the group is touched)
#define WT_G(R, kt, i)                                                               \
  do {                                                                               \
    const int kk_ = (kt) * BK;                                                       \
    const int vr_ = min(max(nr - kk_, 0), BK);                                       \
    const int na_ = __builtin_amdgcn_readfirstlane(vr_ * lda * 2);                   \
    const int nb_ = __builtin_amdgcn_readfirstlane(vr_ * ldb * 2);                   \
    const __amdgpu_buffer_rsrc_t ra_ = __builtin_amdgcn_make_buffer_rsrc(            \
        (void*)(A + (int64_t)(r0 + kk_) * lda), (short)0, na_, 0x00020000);           \
    const __amdgpu_buffer_rsrc_t rb_ = __builtin_amdgcn_make_buffer_rsrc(            \
        (void*)(B + (int64_t)(r0 + kk_) * ldb), (short)0, nb_, 0x00020000);           \
    if ((i) == 0) R.v0 = __builtin_amdgcn_raw_buffer_load_b128(ra_, ao, 0, 0);       \
    if ((i) == 1) R.v1 = __builtin_amdgcn_raw_buffer_load_b128(ra_, ao + astep, 0, 0); \
    if ((i) == 2) R.v2 = __builtin_amdgcn_raw_buffer_load_b128(ra_, ao + 2 * astep, 0, 0); \
    if ((i) == 3) R.v3 = __builtin_amdgcn_raw_buffer_load_b128(ra_, ao + 3 * astep, 0, 0); \
    if ((i) == 4) R.v4 = __builtin_amdgcn_raw_buffer_load_b128(rb_, bo, 0, 0);       \
    if ((i) == 5) R.v5 = __builtin_amdgcn_raw_buffer_load_b128(rb_, bo + bstep, 0, 0); \
    if ((i) == 6) R.v6 = __builtin_amdgcn_raw_buffer_load_b128(rb_, bo + 2 * bstep, 0, 0); \
    if ((i) == 7) R.v7 = __builtin_amdgcn_raw_buffer_load_b128(rb_, bo + 3 * bstep, 0, 0); \
  } while (0)
#define WT_W(R, st, i)                                                               \
  do {                                                                               \
    u32x4* d_ = smem + (st) * STAGE + wslot;                                         \
    if ((i) == 0) d_[0] = R.v0;                                                      \
    if ((i) == 1) d_[16 * TC] = R.v1;                                                \
    if ((i) == 2) d_[32 * TC] = R.v2;                                                \
    if ((i) == 3) d_[48 * TC] = R.v3;                                                \
    if ((i) == 4) d_[HALF] = R.v4;                                                   \
    if ((i) == 5) d_[HALF + 16 * TC] = R.v5;                                         \
    if ((i) == 6) d_[HALF + 32 * TC] = R.v6;                                         \
    if ((i) == 7) d_[HALF + 48 * TC] = R.v7;                                         \
  } while (0)
#define WT_R(F, st, s4, f)                                                           \
  F[f] = lds_tr_frag(smem, (uint32_t)((st) * STAGE * 16 + (s4) * 4096) +             \
                               ((f) < 2 ? fa[(f) & 1] : fb[(f) & 1]))
#define WT_M(F, q)                                                                   \
  acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[2 + ((q) >> 1)], F[(q) & 1], acc[q], 0, 0, 0)
  // one K step from stage st (as the forward kernel's: four sub-steps of four
  // MFMAs, each followed by a fragment read of the next sub-step; global loads
  // of set RG (step KL) in sub-steps 0 / 1, LDS writes of set RW to the other
  // stage in sub-steps 2 / 3)
#define WT_STEP(st, RG, KL, LD, RW, WR)                                              \
  do {                                                                               \
    WT_R(fr0, st, 0, 0); WT_R(fr0, st, 0, 2); WT_R(fr0, st, 0, 1);                   \
    WT_R(fr0, st, 0, 3); WT_SB();                                                    \
    _Pragma("unroll") for (int k_ = 0; k_ < 4; ++k_) {                               \
      WT_M(fr0, k_); WT_SB(); WT_R(fr1, st, 1, kRO[k_]); WT_SB();                    \
      if (LD) { WT_G(RG, KL, 2 * k_); WT_G(RG, KL, 2 * k_ + 1); }                    \
      WT_SB();                                                                       \
    }                                                                                \
    _Pragma("unroll") for (int k_ = 0; k_ < 4; ++k_) {                               \
      WT_M(fr1, k_); WT_SB(); WT_R(fr0, st, 2, kRO[k_]); WT_SB();                    \
    }                                                                                \
    _Pragma("unroll") for (int k_ = 0; k_ < 4; ++k_) {                               \
      WT_M(fr0, k_); WT_SB(); WT_R(fr1, st, 3, kRO[k_]); WT_SB();                    \
      if (WR) WT_W(RW, 1 - (st), k_);                                                \
      WT_SB();                                                                       \
    }                                                                                \
    _Pragma("unroll") for (int k_ = 0; k_ < 4; ++k_) {                               \
      WT_M(fr1, k_); WT_SB();                                                        \
      if (WR) WT_W(RW, 1 - (st), 4 + k_);                                            \
      WT_SB();                                                                       \
    }                                                                                \
  } while (0)

  float* __restrict__ Cg = g < E ? C + (int64_t)g * M * N : Cs;
  f32x4* st4 = reinterpret_cast<f32x4*>(smem);
  const int qo = tid & 31;   // 16-byte chunk of a row segment that this thread stores
#pragma unroll
  for (int i = 0; i < 8; ++i) WT_G(r0v, 0, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) WT_G(r1v, 1, i);
  // n tiles n0, n0 + 128, ... of the run; the first two K steps of the next
  // tile are loaded before this tile's stores, so they arrive while the
  // stores drain
  for (int it = 0; it < ntb; ++it) {
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k4][r] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) WT_W(r0v, 0, i);
  __syncthreads();
  for (int kt = 0; kt < len - 2; kt += 2) {
    WT_STEP(0, r0v, kt + 2, true, r1v, true);
    __syncthreads();
    WT_STEP(1, r1v, kt + 3, true, r0v, true);
    __syncthreads();
  }
  WT_STEP(0, r0v, 0, false, r1v, true);
  __syncthreads();
  WT_STEP(1, r1v, 0, false, r0v, false);
  // lane (fr, fk) of accumulator (i, j) holds row wm 64 + 32 i + fr and
  // columns wn 64 + 32 j + 8 qd + 4 fk .. + 3 of the tile. The float32 tile
  // (64 KB, both stages) leaves through LDS, 16-byte chunk q of row m at
  // q ^ (m & 31), so that each store instruction writes whole 512-byte row
  // segments of C_g.
  __syncthreads();   // every wave is done reading the operand stages
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = wm * 64 + i * 32 + fr;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const f32x4 v = {acc[i + 2 * j][qd * 4 + 0], acc[i + 2 * j][qd * 4 + 1],
                         acc[i + 2 * j][qd * 4 + 2], acc[i + 2 * j][qd * 4 + 3]};
        const int q = wn * 16 + j * 8 + qd * 2 + fk;
        st4[m * 32 + (q ^ (m & 31))] = v;
      }
  }
  __syncthreads();
  if (it + 1 < ntb) {
    bo += BN * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) WT_G(r0v, 0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) WT_G(r1v, 1, i);
  }
  float* crow = Cg + (int64_t)m0 * N + n0 + qo * 4;
#pragma unroll 4
  for (int p = 0; p < 16; ++p) {
    const int m = p * 8 + (tid >> 5);
    __builtin_nontemporal_store(st4[m * 32 + (qo ^ (m & 31))], reinterpret_cast<f32x4*>(crow + (int64_t)m * N));
  }
  n0 += BN;
  __syncthreads();   // the staged tile has been read before stage 0 is refilled
  }
#undef WT_SB
#undef WT_G
#undef WT_W
#undef WT_R
#undef WT_M
#undef WT_STEP
}

// The weight gradient of gemm_wgrad_tn_kernel on 256 x 256 tiles: one block
// of four waves per CU, each wave 128 x 128 with its 256 float32 accumulators
// in the accumulation registers (half the LDS bytes per FLOP of the 128 x 128
// tile, whose fragment reads bound it). Operands go global -> LDS directly
// (buffer_load ... lds, 16 bytes per lane): a stage holds the A and the B
// tile, 64 rows x 512 bytes each (32 KB), in two LDS arrays of two stages;
// waves 0 / 1 load A rows 0..31 / 32..63, waves 2 / 3 the B rows, two rows per
// instruction. Lane l of an instruction lands at physical chunk l & 31 of its
// row, which holds logical chunk (l & 31) ^ 4 (row & 3), so the transposed
// fragment reads (lds_tr_frag, 512-byte rows) see four rows in four distinct
// bank groups. Each K step's buffer descriptors span only its rows inside the
// group, so rows past the group's end land in LDS as zeros. One barrier per K
// step, as in gemm_bf16_big_kernel: the step's last sub-step runs from
// registers while the next step's first fragments are read and the loads of
// the step after go to the other stage.
__global__ __launch_bounds__(256, 1) void gemm_wgrad_tn_big_kernel(
    const bf16* __restrict__ A, int lda, const bf16* __restrict__ B, int ldb,
    const int32_t* __restrict__ so, int G, int E, int M, int N, float* __restrict__ C,
    float* __restrict__ Cs) {
  constexpr int BM = 256, BN = 256, BK = 64, TC = 32;   // 32 chunks of 16 B per LDS row
  constexpr int HALF = BK * TC;                          // chunks of one operand tile (32 KB)
  constexpr int STAGE = 2 * HALF;
  constexpr int GROUP_M = 8;
  __shared__ u32x4 sm0[STAGE], sm1[STAGE];
  const int mtn = M / BM, ntn = N / BN, per = mtn * ntn;
  const int tiles = G * per;
  const int b = blockIdx.x;
  if (b >= tiles) return;
  const int t8 = tiles & ~7;
  const int t = b < t8 ? (b & 7) * (t8 >> 3) + (b >> 3) : b;
  const int g = t / per;
  const int in = t - g * per;
  const int grp = in / (GROUP_M * ntn);
  const int first_m = grp * GROUP_M;
  const int gm = min(mtn - first_m, GROUP_M);
  const int in2 = in - grp * GROUP_M * ntn;
  const int m0 = (first_m + in2 % gm) * BM;
  const int n0 = (in2 / gm) * BN;
  const int r0 = __builtin_amdgcn_readfirstlane(so[g]);
  const int nr = __builtin_amdgcn_readfirstlane(so[g + 1]) - r0;   // the group's rows
  int nk = (nr + BK - 1) / BK;   // K steps, made even and at least 2
  nk = nk < 2 ? 2 : (nk + 1) & ~1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31;
  const int fk = lane >> 5;

  // this wave's operand (uniform): A for waves 0 / 1, B for 2 / 3
  const bf16* X = wave < 2 ? A : B;
  const int ld = wave < 2 ? lda : ldb;
  const int c0 = wave < 2 ? m0 : n0;
  uint32_t doff[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 32 * (wave & 1) + 2 * i + (lane >> 5);
    const int lch = (lane & 31) ^ ((row & 3) << 2);
    doff[i] = (uint32_t)(row * ld + c0 + lch * 8) * 2u;
  }
  const int dl = wave * 1024;   // this wave's first chunk in a stage
  // fragment byte offsets in a stage: A sub-tile i, B sub-tile j (+ 8192 per
  // 16-row sub-step)
  uint32_t fo[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int x = lane & 15, hq = (lane >> 4) & 1;
    const int krow = 8 * fk + (x >> 2);
    const int ch = (f < 4 ? wm * 16 + f * 4 : wn * 16 + (f - 4) * 4) + 2 * hq + ((x & 3) >> 1);
    fo[f] = (uint32_t)(((f < 4 ? 0 : HALF) + krow * TC + (ch ^ ((krow & 3) << 2))) * 16 + (x & 1) * 8);
  }
  constexpr int kRO[8] = {0, 4, 1, 2, 3, 5, 6, 7};   // read order: A0 B0 A1 A2 A3 B1 B2 B3

  bf16x8 fa[8], fb[8];   // [0..3]: A sub-tiles, [4..7]: B sub-tiles
  f32x16 acc[16];        // acc[i + 4 j] = B sub-tile j times A sub-tile i
#pragma unroll
  for (int q = 0; q < 16; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;

#define WB_SB() __builtin_amdgcn_sched_barrier(0)
#define WB_SM(x) ((x) == 0 ? sm0 : sm1)
#define WB_LDS(p) ((__attribute__((address_space(3))) void*)(p))
  // the buffer descriptor of K step kt (scalar: rows of the step inside the group)
#define WB_RSRC(kt)                                                                  \
  __builtin_amdgcn_make_buffer_rsrc(                                                 \
      (void*)(X + (int64_t)(r0 + (kt) * BK) * ld), (short)0,                         \
      __builtin_amdgcn_readfirstlane(min(max(nr - (kt) * BK, 0), BK) * ld * 2), 0x00020000)
#define WB_D(x, rs, i)                                                               \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, WB_LDS(WB_SM(x) + dl + (i) * 64), 16, doff[i], 0, 0, 0)
#define WB_R(F, x, s4, f)                                                            \
  F[f] = lds_tr_frag<512>(WB_SM(x), (uint32_t)((s4) * 8192) + fo[f])
#define WB_M(F, q)                                                                   \
  acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[4 + ((q) >> 2)], F[(q) & 3], acc[q], 0, 0, 0)
  // wait for this wave's direct-to-LDS loads (vmcnt 0, expcnt and lgkmcnt free)
#define WB_WAIT_LOADS() __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8))
  // one sub-step: 16 MFMAs, the first 8 followed by a fragment read of the next
  // sub-step (RD), every second one by one of 8 loads d0 .. d0 + 7 of step KN
  // into the other stage (LD)
#define WB_SUB(FC, FN, x, s4n, RD, LD, rs, d0)                                       \
  _Pragma("unroll") for (int q_ = 0; q_ < 16; ++q_) {                                \
    WB_M(FC, q_); WB_SB();                                                           \
    if ((RD) && q_ < 8) WB_R(FN, x, s4n, kRO[q_]);                                   \
    if ((LD) && (q_ & 1)) WB_D(1 - (x), rs, (d0) + (q_ >> 1));                       \
    WB_SB();                                                                         \
  }
  // phase k: sub-step 3 of step k - 1 while step k's first fragments are read
  // from stage x and step KN's loads go to the other stage, then sub-steps
  // 0..2 of step k, the wait for this wave's loads and the barrier
#define WB_PHASE(x, KN, LD)                                                          \
  do {                                                                               \
    const __amdgpu_buffer_rsrc_t rs_ = WB_RSRC(KN);                                  \
    WB_SUB(fb, fa, x, 0, true, LD, rs_, 0)                                           \
    WB_SUB(fa, fb, x, 1, true, LD, rs_, 8)                                           \
    WB_SUB(fb, fa, x, 2, true, false, rs_, 0)                                        \
    WB_SUB(fa, fb, x, 3, true, false, rs_, 0)                                        \
    WB_WAIT_LOADS();                                                                 \
    __builtin_amdgcn_s_barrier();                                                    \
    WB_SB();                                                                         \
  } while (0)

  {
    const __amdgpu_buffer_rsrc_t rs0 = WB_RSRC(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) WB_D(0, rs0, i);
  }
  WB_WAIT_LOADS();
  __builtin_amdgcn_s_barrier();
  WB_SB();
  // phase 0: no previous step; all 16 loads of step 1 go out in sub-step 0
#pragma unroll
  for (int f = 0; f < 8; ++f) WB_R(fa, 0, 0, kRO[f]);
  WB_SB();
  {
    const __amdgpu_buffer_rsrc_t rs1 = WB_RSRC(1);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      WB_M(fa, q); WB_SB();
      if (q < 8) WB_R(fb, 0, 1, kRO[q]);
      WB_D(1, rs1, q);
      WB_SB();
    }
    WB_SUB(fb, fa, 0, 2, true, false, rs1, 0)
    WB_SUB(fa, fb, 0, 3, true, false, rs1, 0)
  }
  WB_WAIT_LOADS();
  __builtin_amdgcn_s_barrier();
  WB_SB();
  // phases 1 .. nk - 1 (nk even)
  for (int kt = 1; kt < nk - 1; kt += 2) {
    WB_PHASE(1, kt + 1, true);
    WB_PHASE(0, kt + 2, true);
  }
  WB_PHASE(1, 0, false);
  // sub-step 3 of the last step
#pragma unroll
  for (int q = 0; q < 16; ++q) { WB_M(fb, q); WB_SB(); }
#undef WB_SB
#undef WB_SM
#undef WB_LDS
#undef WB_RSRC
#undef WB_D
#undef WB_R
#undef WB_M
#undef WB_WAIT_LOADS
#undef WB_SUB
#undef WB_PHASE

  // lane (fr, fk) of accumulator (i, j) holds row wm 128 + 32 i + fr and
  // columns wn 128 + 32 j + 8 qd + 4 fk .. + 3 of the tile. The float32 tile
  // (256 KB) leaves through LDS in two halves of 128 rows (the waves with
  // wm = 0, then wm = 1, stage theirs: rows 0..63 of the half in sm0, 64..127
  // in sm1, 16-byte chunk q of row m at q ^ (m & 31)), so that each store
  // instruction writes whole 1 KB row segments of C_g.
  float* __restrict__ Cg = g < E ? C + (int64_t)g * M * N : Cs;
  f32x4* st_lo = reinterpret_cast<f32x4*>(sm0);
  f32x4* st_hi = reinterpret_cast<f32x4*>(sm1);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = i * 32 + fr;   // row of the half
        f32x4* st = i < 2 ? st_lo : st_hi;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x16& a = acc[i + 4 * j];
            const f32x4 v = {a[qd * 4 + 0], a[qd * 4 + 1], a[qd * 4 + 2], a[qd * 4 + 3]};
            const int q = wn * 32 + j * 8 + qd * 2 + fk;
            st[(m & 63) * 64 + (q ^ (m & 31))] = v;
          }
      }
    }
    __syncthreads();
    const int q = tid & 63;
    float* crow = Cg + (int64_t)(m0 + half * 128) * N + n0 + q * 4;
#pragma unroll 4
    for (int p = 0; p < 16; ++p) {
      const int m = p * 4 + (tid >> 6);
      *reinterpret_cast<f32x4*>(crow + (int64_t)m * N) = st_lo[m * 64 + (q ^ (m & 31))];
    }
#pragma unroll 4
    for (int p = 0; p < 16; ++p) {
      const int m = p * 4 + (tid >> 6);
      *reinterpret_cast<f32x4*>(crow + (int64_t)(64 + m) * N) = st_hi[m * 64 + ((q ^ (m & 31)))];
    }
    __syncthreads();
  }
}

// Grouped GEMM on the full 256-row tiles of each group (part 1 of the row
// space): 256 x 256 output tiles (SwiGLU: 256 x 128 of W1 and of W3), one block
// of four waves per CU, each wave 128 x 128 (SwiGLU 128 x 64 per operand) with
// its 256 float32 accumulators in the accumulation registers. A 256 x 256 tile
// needs half the bytes per FLOP of a 128 x 128 one, which keeps the CU's
// address unit below saturation. Operands go global -> LDS directly
// (buffer_load ... lds, 16 bytes per lane), 64-deep K steps, two stages of
// 512 rows x 128 B (A rows, then B rows) held in two separate LDS arrays so
// that the compiler can tell the loads into one stage from the fragment reads
// of the other. There is one barrier per K step, placed after the last
// fragment read of the step's stage rather than at the step's end: after it,
// the step's last 16 MFMAs run from registers while the next step's first
// fragments are read and its loads are issued, so no wave waits on LDS right
// after a barrier.
// Lane l of a load lands at LDS row (l >> 3) of its 8-row group and physical
// chunk l & 7, which holds logical chunk (l & 7) ^ ((row >> 1) & 7): the
// same conflict-free layout as the 128 x 128 kernel. The epilogue adds the
// bias, applies the activation, stages the bf16 tile in LDS and writes whole
// 512-byte row segments.
template <int EPI, bool HAS_BIAS, bool KMB = false>
__global__ __launch_bounds__(256, 1) void gemm_bf16_big_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* __restrict__ W3,
    const float* __restrict__ bias, const bf16* __restrict__ Ws, const bf16* __restrict__ Ws3,
    const float* __restrict__ bias_s, int E, int G, const int32_t* __restrict__ offsets,
    int rows_max, bf16* __restrict__ C, int N, int K, const int32_t* __restrict__ arows,
    uint32_t a_bytes, int skip_rows, int skip_last, int ksplit) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  static_assert(!KMB || !GATED, "K-major weights: ungated GEMMs");
  constexpr int BM = 256, BK = 64, CH = BK / 8;   // 8 chunks of 16 B per LDS row
  constexpr int NB = GATED ? 2 : 1;
  constexpr int BN = GATED ? 128 : 256;           // columns per B operand = output columns
  constexpr int WN = BN / 2;                       // per wave, per operand
  constexpr int TN = WN / 32;                      // 4 (SwiGLU 2)
  constexpr int STAGE = 512 * CH;                  // u32x4 per stage (64 KB)
  constexpr int GROUP_M = 8;
  constexpr int CQ = BN / 8;                       // 16-byte chunks per output row
  static_assert(NB * TN == 4, "four B fragments per sub-step");
  static_assert(128 * CQ <= STAGE, "half of the output tile fits one stage");
  __shared__ u32x4 sm0[STAGE], sm1[STAGE];
  __shared__ uint32_t pf_lds[512];   // landing area of the L2 prefetches, never read

  TileSpace ts;
  tile_space_init(ts, offsets, G, rows_max, BM, 1, BM, skip_rows, skip_last);
  const int mtiles = __builtin_amdgcn_readfirstlane(ts.total);
  const int ntn = N / BN;
  const int tiles = mtiles * ntn;
  const int b = blockIdx.x;
  if (b >= tiles) return;
  const int t8 = tiles & ~7;
  const int t = b < t8 ? (b & 7) * (t8 >> 3) + (b >> 3) : b;
  const int per_group = GROUP_M * ntn;
  const int grp = t / per_group;
  const int first_m = grp * GROUP_M;
  const int in = t - grp * per_group;
  const int gm = min(mtiles - first_m, GROUP_M);
  const int mt = first_m + in % gm;
  const int nt = in / gm;
  int g, row0, nrows;
  tile_lookup(ts, mt, BM, g, row0, nrows);
  g = __builtin_amdgcn_readfirstlane(g);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  nrows = __builtin_amdgcn_readfirstlane(nrows);   // BM: part 1 has only full tiles
  const int n0 = nt * BN;
  // KMB: W_g [K][N] at W + g ksplit N for K rows below ksplit, W3_g for the
  // rest (as gemm_bf16_kernel's KMB)
  const bf16* Wg = KMB ? (g < E ? W + (int64_t)g * ksplit * N : Ws)
                       : (g < E ? W + (int64_t)g * N * K : Ws);
  const bf16* W3g = KMB ? (g < E ? (W3 ? W3 + (int64_t)g * ksplit * N : Wg) : (Ws3 ? Ws3 : Wg))
                        : (GATED ? (g < E ? W3 + (int64_t)g * N * K : Ws3) : Wg);
  const float* bg = HAS_BIAS ? (g < E ? bias + (int64_t)g * N : bias_s) : nullptr;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31;
  const int fk = lane >> 5;

  // Direct-to-LDS loads: wave w fills stage rows 128 w .. 128 w + 127 (waves 0
  // and 1: A rows; 2 and 3: W rows n0 .., or W1 then W3 rows for SwiGLU), 8 rows
  // per instruction i; (row >> 1) & 7 = (4 (i & 1) + (lane >> 4)) & 7.
  // A rows: row row0 + r of A, or, with arows, row arows[row0 + r] (the
  // expert-sorted gather of token rows, fused here)
  const int pc = lane & 7, lq = lane >> 4;
  // Each wave reads through its own buffer resource (wave-uniform base and
  // size) with 32-bit lane offsets; the K step enters as the scalar offset.
  // Buffer loads, unlike flat/global ones, are not taken by the compiler as
  // possible LDS accesses, so its LDS-read waits stay exact.
  const char* wbase;
  uint32_t wbytes;
  if (wave < 2) {
    wbase = arows ? reinterpret_cast<const char*>(A)
                  : reinterpret_cast<const char*>(A + (int64_t)(row0 + wave * 128) * K);
    wbytes = arows ? a_bytes : 128u * (uint32_t)K * 2u;
  } else if (KMB) {
    wbase = reinterpret_cast<const char*>(Wg + n0);   // per K step: MOE_KRS
    wbytes = 0u;
  } else {
    wbase = reinterpret_cast<const char*>(GATED ? (wave == 2 ? Wg : W3g) + (int64_t)n0 * K
                                                : Wg + (int64_t)(n0 + (wave - 2) * 128) * K);
    wbytes = 128u * (uint32_t)K * 2u;
  }
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, (int)wbytes, 0x00020000);
  uint32_t doff[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rl = 8 * i + (lane >> 3);
    const uint32_t rowoff = wave < 2 && arows ? (uint32_t)arows[row0 + wave * 128 + rl] * (uint32_t)K * 2u
                                              : (uint32_t)rl * (uint32_t)K * 2u;
    doff[i] = rowoff + (uint32_t)(pc ^ ((4 * (i & 1) + lq) & 7)) * 16u;
    if (KMB && wave >= 2) {
      // K-major W: K rows 32 (wave - 2) + 2 i + lane / 32 of the step, 512 bytes
      // (256 columns) each, physical chunk lane & 31 holding logical chunk
      // (lane & 31) ^ 4 (row & 3)
      const int kr = 32 * (wave - 2) + 2 * i + (lane >> 5);
      doff[i] = (uint32_t)(kr * N + ((lane & 31) ^ ((kr & 3) << 2)) * 8) * 2u;
    }
  }
  // KMB: the buffer descriptor of K step kt for the W waves (64 K rows of W_g,
  // or of W3_g from ksplit on, columns n0 ..; scalar)
#define MOE_KRS(kt)                                                                  \
  __builtin_amdgcn_make_buffer_rsrc(                                                 \
      (void*)(((kt) * BK < ksplit ? Wg + (int64_t)(kt) * BK * N                      \
                                  : W3g + (int64_t)((kt) * BK - ksplit) * N) + n0),  \
      (short)0, BK * N * 2, 0x00020000)
  const int dl = wave * 128 * CH;
  // L2 prefetch: in phase k (below), which loads step k + 1, each lane also
  // loads one dword of the 128-byte K chunk of step k + 3 for rows l and
  // l + 64 of its wave's 128 rows, so the loads of that step, issued in phase
  // k + 2, find their lines in L2 instead of waiting on HBM. The dwords land in a small LDS area
  // that is never read (a load with no register result, so nothing has to
  // consume it and the waits stay exact).
  uint32_t pfo[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rl = lane + 64 * j;
    pfo[j] = wave < 2 && arows ? (uint32_t)arows[row0 + wave * 128 + rl] * (uint32_t)K * 2u
                               : (uint32_t)rl * (uint32_t)K * 2u;
    // KMB W waves: one dword of each 128-byte line of the wave's 32 K rows
    if (KMB && wave >= 2)
      pfo[j] = (uint32_t)((32 * (wave - 2) + (rl >> 2)) * N + (rl & 3) * 64) * 2u;
  }
  const int nk = K / BK;   // K is a multiple of 256, so nk >= 4 and even

  // KMB: byte offsets of the W fragments (f = 4..7, W sub-tile f - 4) in a
  // stage, read transposed (+ 8192 per 16-row sub-step)
  uint32_t fo[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int x = lane & 15, hq = (lane >> 4) & 1;
    const int krow = 8 * fk + (x >> 2);
    const int ch = wn * 16 + jb * 4 + 2 * hq + ((x & 3) >> 1);
    fo[jb] = (uint32_t)((256 * CH + krow * 32 + (ch ^ ((krow & 3) << 2))) * 16 + (x & 1) * 8);
  }
  int fbase[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int jb = f - 4;
    const int row = f < 4 ? wm * 128 + f * 32 + fr
                          : 256 + (jb / TN) * BN + wn * WN + (jb % TN) * 32 + fr;
    fbase[f] = row * CH;
  }
  const int rsw = (fr >> 1) & 7;
  int cidx[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) cidx[s4] = (s4 * 2 + fk) ^ rsw;
  constexpr int kRO[8] = {0, 4, 1, 2, 3, 5, 6, 7};   // read order: A0 B0 A1 A2 A3 B1 B2 B3

  bf16x8 fa[8], fb[8];
  f32x16 acc[16];   // acc[i + 4 jb] = A sub-tile i times B sub-tile jb
#pragma unroll
  for (int q = 0; q < 16; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;

#define MOE_SB() __builtin_amdgcn_sched_barrier(0)
#define MOE_SM(x) ((x) == 0 ? sm0 : sm1)
#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define MOE_D(x, kt, i)                                                              \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(KMB && wave >= 2 ? MOE_KRS(kt) : rsrc,   \
                                           MOE_LDS(MOE_SM(x) + dl + (i) * 8 * CH), 16, doff[i], \
                                           KMB && wave >= 2 ? 0u : (uint32_t)(kt) * (BK * 2), 0, 0)
#define MOE_R(F, x, s4, f)                                                           \
  do {                                                                               \
    if (KMB && (f) >= 4)                                                             \
      F[f] = lds_tr_frag<512>(MOE_SM(x), (uint32_t)((s4) * 8192) + fo[(f) & 3]);    \
    else                                                                             \
      F[f] = __builtin_bit_cast(bf16x8, MOE_SM(x)[fbase[f] + cidx[s4]]);            \
  } while (0)
#define MOE_M(F, q)                                                                  \
  acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[4 + ((q) >> 2)], F[(q) & 3], acc[q], 0, 0, 0)
  // wait for this wave's direct-to-LDS loads (vmcnt 0, expcnt and lgkmcnt free)
#define MOE_WAIT_LOADS() __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8))
  // the same but for the two prefetches issued last (vmcnt 2)
#define MOE_WAIT_LOADS_PF() __builtin_amdgcn_s_waitcnt(2 | (7 << 4) | (15 << 8))
#define MOE_PF(kt)                                                                   \
  do {                                                                               \
    const bool kw_ = KMB && wave >= 2;                                               \
    const __amdgpu_buffer_rsrc_t r_ = kw_ ? MOE_KRS(min((kt), nk - 1)) : rsrc;      \
    const uint32_t o_ = kw_ ? 0u : (uint32_t)min((kt), nk - 1) * (BK * 2);           \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, MOE_LDS(pf_lds + wave * 128), 4, pfo[0], o_, 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r_, MOE_LDS(pf_lds + wave * 128 + 64), 4, pfo[1], o_, 0, 0); \
  } while (0)
  // One K step from stage x: 64 MFMAs in four sub-steps; each MFMA is
  // followed by one fragment read of the next sub-step, and every third of
  // the first 48 by one of the 16 loads of step KL into the other stage (LD):
  // spread out, the loads do not queue up in the address unit and hold back
  // the MFMAs behind them, and they still have a quarter step to land.
  // Phase k (between the barriers that end phases k - 1 and k): sub-step 3 of
  // step k - 1 (its fragments are already in registers) while the first
  // fragments of step k are read from stage x = k % 2 and the loads of step
  // k + 1 go to the other stage (both are safe after the previous barrier:
  // step k's loads have landed and every wave has read all of step k - 1 it
  // needs); then sub-steps 0..2 of step k, the wait for this wave's loads and
  // the barrier. No wave waits on LDS right after a barrier.
#define MOE_SUB(FC, FN, x, s4n, RD, LD, KN, d0)                                      \
  _Pragma("unroll") for (int q_ = 0; q_ < 16; ++q_) {                                \
    MOE_M(FC, q_); MOE_SB();                                                         \
    if ((RD) && q_ < 8) MOE_R(FN, x, s4n, kRO[q_]);                                  \
    if ((LD) && (q_ & 1)) MOE_D(1 - (x), KN, (d0) + (q_ >> 1));                      \
    MOE_SB();                                                                        \
  }
#define MOE_PHASE(x, KN, LD)                                                         \
  do {                                                                               \
    MOE_SUB(fb, fa, x, 0, true, LD, KN, 0)                                           \
    MOE_SUB(fa, fb, x, 1, true, LD, KN, 8)                                           \
    if (LD) { MOE_PF((KN) + 2); MOE_SB(); }                                          \
    MOE_SUB(fb, fa, x, 2, true, false, 0, 0)                                         \
    MOE_SUB(fa, fb, x, 3, true, false, 0, 0)                                         \
    if (LD) MOE_WAIT_LOADS_PF(); else MOE_WAIT_LOADS();                              \
    __builtin_amdgcn_s_barrier();                                                    \
    MOE_SB();                                                                        \
  } while (0)

#pragma unroll
  for (int i = 0; i < 16; ++i) MOE_D(0, 0, i);
  MOE_PF(2);
  MOE_WAIT_LOADS_PF();
  __builtin_amdgcn_s_barrier();
  MOE_SB();
  // phase 0: no previous step; all 16 loads of step 1 go out in sub-step 0
#pragma unroll
  for (int f = 0; f < 8; ++f) MOE_R(fa, 0, 0, kRO[f]);
  MOE_SB();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    MOE_M(fa, q); MOE_SB();
    if (q < 8) MOE_R(fb, 0, 1, kRO[q]);
    MOE_D(1, 1, q);
    MOE_SB();
  }
  MOE_PF(3);
  MOE_SB();
  MOE_SUB(fb, fa, 0, 2, true, false, 0, 0)
  MOE_SUB(fa, fb, 0, 3, true, false, 0, 0)
  MOE_WAIT_LOADS_PF();
  __builtin_amdgcn_s_barrier();
  MOE_SB();
  // phases 1 .. nk - 1 (nk is a multiple of 4)
  for (int kt = 1; kt < nk - 1; kt += 2) {
    MOE_PHASE(1, kt + 1, true);
    MOE_PHASE(0, kt + 2, true);
  }
  MOE_PHASE(1, 0, false);
  // sub-step 3 of the last step
#pragma unroll
  for (int q = 0; q < 16; ++q) { MOE_M(fb, q); MOE_SB(); }
#undef MOE_SB
#undef MOE_D
#undef MOE_R
#undef MOE_M
#undef MOE_WAIT_LOADS
#undef MOE_WAIT_LOADS_PF
#undef MOE_PF
#undef MOE_LDS
#undef MOE_SUB
#undef MOE_PHASE
#undef MOE_KRS

  // Epilogue: rows 0..127 of the tile are staged in sm0, rows 128..255 in sm1
  // (wave row half wm); chunk q of row m at q ^ (m & 15). Every fragment read
  // came before the last barrier and no load is in flight, so the stages are
  // free.
  uint2* st8 = reinterpret_cast<uint2*>(wm ? sm1 : sm0);
#pragma unroll
  for (int jx = 0; jx < TN; ++jx) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const float4 bq = HAS_BIAS ? *reinterpret_cast<const float4*>(bg + n0 + wn * WN + jx * 32 + qd * 8 + fk * 4)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = i * 32 + fr;   // row within this wave's half
        const f32x16& a1 = acc[i + 4 * jx];
        const float z[4] = {a1[qd * 4 + 0] + bq.x, a1[qd * 4 + 1] + bq.y, a1[qd * 4 + 2] + bq.z,
                            a1[qd * 4 + 3] + bq.w};
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = epilogue_bf16<EPI>(z[e], GATED ? acc[i + 4 * (TN + jx)][qd * 4 + e] : 0.f);
        uint2 uu;
        uu.x = pack_bf16x2(v[0], v[1]);
        uu.y = pack_bf16x2(v[2], v[3]);
        const int q = wn * (WN / 8) + jx * 4 + qd;
        st8[(m * CQ + (q ^ (m & 15))) * 2 + fk] = uu;
      }
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int p = 0; p < BM * CQ / 256; ++p) {
    const int idx = p * 256 + tid;
    const int m = idx / CQ, q = idx % CQ;
    const u32x4 v = (m >> 7 ? sm1 : sm0)[(m & 127) * CQ + (q ^ (m & 15))];
    if (m < nrows) *reinterpret_cast<u32x4*>(C + (int64_t)(row0 + m) * N + n0 + q * 8) = v;
  }
}

// ------------------------------------------------------------------ weight-streaming grouped GEMM
// Groups with few rows (the fine-grained experts of a DeepSeek-V3-shaped layer
// hold tens to a few hundred rows each) make the grouped GEMM a stream of the
// weights: each weight byte feeds only that many rows, below the ridge point of
// the chip, so the kernel must read every weight byte once, at full HBM rate.
// Here a block takes all rows of one group (in equal parts of at most 256
// rows) against one slab of 256 weight rows (SwiGLU: 128 rows of W1 and the
// same 128 rows of W3), and each wave owns 64 of those weight rows (32 of W1 +
// 32 of W3) for the whole K loop. Per 64-deep K step:
//   * each wave loads its weight rows into registers, three steps ahead, every
//     load instruction covering eight whole 128-byte lines (lane l: row l / 8,
//     16-byte chunk l % 8), with the non-temporal cache policy (read once):
//     HBM delivers whole lines per instruction at about 6-7 TB/s, where the
//     MFMA fragment layout loaded straight into registers (32 rows x 32 bytes
//     per instruction) reaches about 4 TB/s. When its step comes, the wave
//     stores the rows into its own LDS area and reads them back as fragments
//     (each weight byte crosses LDS once, with no barrier between waves);
//   * the group's token rows (gathered through arows for GEMM 1) go global ->
//     LDS directly (buffer_load ... lds), four stages, three steps ahead,
//     cached (the group's other slabs read the same rows), read by every wave.
// v_mfma_f32_32x32x16_bf16 takes the weight fragment first, so a lane's
// accumulators hold four consecutive output columns of one row. LDS rows are
// 128 bytes with 16-byte chunk c of row r at c ^ ((r >> 1) & 7), conflict-free
// for the fragment reads. Within a K step, sub-step s of lane half h multiplies
// K elements 32 h + 8 s .. + 7, the same order on both operands.
// Groups of up to 1536 rows take this kernel (measured on one MI355X: the
// DeepSeek-V3-shaped layer's routed experts of 0-527 rows, and the Mixtral-
// shaped layer's experts of about 1024 rows, four parts each, where it beats
// the 256 x 256 tiles); groups of 2048 rows or more (the DeepSpeed-GPT shape,
// the 4096-row shared expert) are faster on the tiled kernels.
// The parts of one slab are consecutive work items and a group's slabs are
// consecutive, and each XCD runs a contiguous range of items, so the slabs of a
// group run side by side on one XCD: its token rows are fetched into that
// XCD's L2 once, and the parts of a group with more than 256 rows (equal in
// size, so they run at the same pace) read the same weight lines at about the
// same time, the second reader finding them in L2.
// Rows per part are rounded up to a multiple of 32 (template MF = 1 .. 8
// fragments of 32 rows) on packed weights, to 64, 128, 192 or 256 (MF = 2, 4,
// 6, 8) on the standard layout; rows past the part's end repeat its last row
// and are not stored.
constexpr int kStreamRows = 256;   // rows per part
constexpr int kStreamMaxRows = 1536;  // groups with more rows use the tiled kernels,
constexpr int kStreamSharedMaxRows = 4096;   // except a shared group of up to this many
constexpr int kStreamLds = 10240;     // u32x4 (160 KB)
// Work items of the streaming GEMM: group g with rows in (0, max_rows]
// ((min_last, max_last] for the last group, g = G - 1) contributes ns slabs x
// ceil(rows / 256) parts. Lane l of every wave holds groups 5 l .. 5 l + 4
// (first row, row count, item count) and the prefix of items before them.
struct StreamSpace {
  int s[5], r[5], n[5];
  int excl, incl, total;
};

__device__ __forceinline__ void stream_space_init(StreamSpace& ss, const int32_t* __restrict__ offsets,
                                                  int G, int rows_max, int max_rows, int min_last,
                                                  int max_last, int ns) {
  constexpr int PER = 5;
  const int lane = threadIdx.x & 63;
  const int g0 = lane * PER;
  int o[PER + 1];
#pragma unroll
  for (int i = 0; i <= PER; ++i) {
    const int gi = g0 + i;
    o[i] = gi <= G ? min(max(offsets[gi], 0), rows_max) : rows_max;
  }
  int sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int gi = g0 + i;
    const int rows = (gi < G && o[i + 1] > o[i]) ? o[i + 1] - o[i] : 0;
    const bool mine = gi == G - 1 ? rows > min_last && rows <= max_last : rows > 0 && rows <= max_rows;
    ss.s[i] = o[i];
    ss.r[i] = mine ? rows : 0;
    ss.n[i] = mine ? (rows + kStreamRows - 1) / kStreamRows * ns : 0;
    sum += ss.n[i];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  ss.incl = incl;
  ss.excl = incl - sum;
  ss.total = __shfl(incl, 63, 64);
}

// Group, first row, row count and slab of item t (< ss.total); uniform over the wave.
__device__ __forceinline__ void stream_lookup(const StreamSpace& ss, int t, int ns, int& g_out,
                                              int& row0_out, int& nrows_out, int& slab_out) {
  constexpr int PER = 5;
  const int lane = threadIdx.x & 63;
  const bool mine = t >= ss.excl && t < ss.incl;
  const int owner = __ffsll((unsigned long long)__ballot(mine)) - 1;
  int g = 0, row0 = 0, nrows = 0, slab = 0;
  if (mine) {
    int acc = ss.excl;
    bool found = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!found && t < acc + ss.n[i]) {
        found = true;
        const int parts = ss.n[i] / ns;
        const int local = t - acc;
        slab = local / parts;
        const int part = local - slab * parts;
        g = lane * PER + i;
        // equal parts (within one row), so that the parts of a slab run at the
        // same pace and read its weight lines at about the same time
        const int lo = part * ss.r[i] / parts, hi = (part + 1) * ss.r[i] / parts;
        row0 = ss.s[i] + lo;
        nrows = hi - lo;
      }
      acc += ss.n[i];
    }
  }
  g_out = __shfl(g, owner, 64);
  row0_out = __shfl(row0, owner, 64);
  nrows_out = __shfl(nrows, owner, 64);
  slab_out = __shfl(slab, owner, 64);
}

// s_waitcnt immediate: vmcnt <= n (0..63), lgkmcnt 0, expcnt not waited for.
__device__ __forceinline__ constexpr int stream_wait_imm(int n) {
  return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4);
}

// Epilogue of the streaming GEMM: lane (fr, fh) of wave w holds row 32 i + fr
// and, of weight fragment j, columns 8 q + 4 fh .. + 3 in registers
// 4 q .. 4 q + 3; bias, activation (SwiGLU: silu(W1 part) * W3 part), bf16
// rounding, stored as 8-byte pieces; rows past mrows are not stored.
template <int EPI, bool HAS_BIAS, int MF>
__device__ __forceinline__ void stream_epilogue(const f32x16 (&acc)[MF][2], const float* __restrict__ bg,
                                                int row0, int mrows, int n0, bf16* __restrict__ C,
                                                int N) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 31, fh = lane >> 5;
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int m = 32 * i + fr;
    if (m >= mrows) continue;
    bf16* crow = C + (int64_t)(row0 + m) * N;
#pragma unroll
    for (int j = 0; j < (GATED ? 1 : 2); ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = (GATED ? n0 + 32 * wave : n0 + 64 * wave + 32 * j) + 8 * q + 4 * fh;
        const float4 bq = HAS_BIAS ? *reinterpret_cast<const float4*>(bg + c)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = epilogue_bf16<EPI>(acc[i][j][4 * q + e] + bb[e], GATED ? acc[i][1][4 * q + e] : 0.f);
        uint2 u;
        u.x = pack_bf16x2(v[0], v[1]);
        u.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(crow + c) = u;
      }
    }
  }
}

// The same epilogue through LDS: the block's output tile (32 MF rows x 256
// columns, SwiGLU 128) is staged in LDS (rows padded by 16 bytes so that the
// 32 rows of one store land in different banks) and written as whole row
// segments, 16 bytes per lane. Starts with a barrier: every wave must be done
// reading the token-row stages it overwrites.
template <int EPI, bool HAS_BIAS, int MF>
__device__ __forceinline__ void stream_epilogue_lds(const f32x16 (&acc)[MF][2], u32x4* __restrict__ smem,
                                                    const float* __restrict__ bg, int row0, int mrows,
                                                    int n0, bf16* __restrict__ C, int N) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  constexpr int BNO = GATED ? 128 : 256;       // output columns of the tile
  constexpr int RB = BNO * 2 + 16;             // bytes per staged row
  static_assert(32 * MF * RB <= kStreamLds * 16, "output tile fits in LDS");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, fh = lane >> 5;
  char* st = reinterpret_cast<char*>(smem);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int m = 32 * i + fr;
#pragma unroll
    for (int j = 0; j < (GATED ? 1 : 2); ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = (GATED ? 32 * wave : 64 * wave + 32 * j) + 8 * q + 4 * fh;   // column in tile
        const float4 bq = HAS_BIAS ? *reinterpret_cast<const float4*>(bg + n0 + cl)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = epilogue_bf16<EPI>(acc[i][j][4 * q + e] + bb[e], GATED ? acc[i][1][4 * q + e] : 0.f);
        uint2 u;
        u.x = pack_bf16x2(v[0], v[1]);
        u.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(st + m * RB + cl * 2) = u;
      }
    }
  }
  __syncthreads();
  constexpr int CPR = BNO / 8;                 // 16-byte chunks per row
#pragma unroll
  for (int p = 0; p < 32 * MF * CPR / 256; ++p) {
    const int idx = p * 256 + tid;
    const int m = idx / CPR, c = idx % CPR;
    if (m < mrows)
      *reinterpret_cast<u32x4*>(C + (int64_t)(row0 + m) * N + n0 + c * 8) =
          *reinterpret_cast<const u32x4*>(st + m * RB + c * 16);
  }
}

// KMB (backward dH and dX, EPI_NONE): the weights are read as stored,
// K-major, C[r, n] = sum_k A[r, k] W_g[k, n], W_g [ksplit][N] for the K steps
// below ksplit and W3g [K - ksplit][N] for the rest (SwiGLU's dX over
// [W1; W3]). Wave w's part of a K step is then 64 K rows x 128 bytes (its 64
// columns): eight whole-line loads of 8 rows each, stored as they arrived
// into the wave's LDS area (16-byte chunk c of row k at c ^ 4 ((k >> 1) & 1)),
// and every weight fragment is two ds_read_b64_tr_b16 (lds_tr_frag) that
// hand lane (fr, fh) column 32 j + fr at the K rows 32 fh + 8 s .. + 7 of
// sub-step s, the rows its token fragment covers. The four rows a 16-lane
// group reads and the two chunk pairs of a 32-lane half fall on 64 distinct
// banks.
template <int EPI, bool HAS_BIAS, int MF, bool KMB = false>
__device__ __forceinline__ int stream_tile(u32x4* __restrict__ smem, const bf16* __restrict__ A,
                                           uint32_t a_bytes, const int32_t* __restrict__ arows,
                                           const bf16* __restrict__ Wg, const bf16* __restrict__ W3g,
                                           const float* __restrict__ bg, int row0, int mrows,
                                           int n0, bf16* __restrict__ C, int N, int K,
                                           int* __restrict__ done, int ksplit = 0) {
  static_assert(!KMB || EPI == EPI_NONE, "K-major streaming: linear epilogue only");
  constexpr bool GATED = EPI == EPI_SWIGLU;
  constexpr int CH = 8;                        // 16-byte chunks per 128-byte LDS row
  constexpr int WAREA = 64 * CH;               // u32x4: one wave's 64 weight rows
  constexpr int ABASE = 4 * WAREA;             // token-row stages after the weight areas
  constexpr int ASTAGE = 32 * MF * CH;         // u32x4 per token-row stage
  constexpr int NW = 8;                        // weight loads per wave per K step
  constexpr int NA = MF;                       // token-row loads per wave per K step
  constexpr int NL = NW + NA;
  static_assert(ABASE + 4 * ASTAGE <= kStreamLds, "LDS");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, fh = lane >> 5;
  const int nk = K / 64;                       // multiple of 4
  const int lr = lane >> 3;                    // row of a load within its 8-row group
  const int lc = lane & 7;                     // 16-byte chunk of a load

  // token rows: wave w loads stage rows 8 (w MF + i) + lr
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)a_bytes, 0x00020000);
  uint32_t aoff[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int rl = 8 * (wave * MF + i) + lr;
    const int r = row0 + min(rl, mrows - 1);
    const uint32_t rowoff = (uint32_t)(arows ? arows[r] : r) * (uint32_t)K * 2u;
    aoff[i] = rowoff + (uint32_t)(lc ^ ((rl >> 1) & 7)) * 16u;
  }
  // weight rows of this wave: fragment j = 32 consecutive rows of W (SwiGLU:
  // j = 0 of W1, j = 1 of W3); load i (fragment i / 4) brings rows 8 (i % 4) + lr
  // of the fragment, chunk lc, into registers, then into the wave's LDS area
  // at row 8 i + lr, chunk lc ^ ((row >> 1) & 7)
  // (KMB: rw0 spans this wave's columns of W_g's ksplit K rows, rw1 those of
  // W3g; load i brings K row 8 i + lr of the step, chunk lc)
  const int kcol = KMB ? n0 + 64 * wave : 0;
  const bf16* wrow0 = KMB ? Wg + kcol
                          : GATED ? Wg + (int64_t)(n0 + 32 * wave) * K
                                  : Wg + (int64_t)(n0 + 64 * wave) * K;
  const bf16* wrow1 = KMB ? (W3g ? W3g : Wg) + kcol
                          : GATED ? W3g + (int64_t)(n0 + 32 * wave) * K
                                  : Wg + (int64_t)(n0 + 64 * wave + 32) * K;
  const int wbytes0 = KMB ? (ksplit * N - kcol) * 2 : 32 * K * 2;
  const int wbytes1 = KMB ? ((W3g ? K - ksplit : ksplit) * N - kcol) * 2 : 32 * K * 2;
  const __amdgpu_buffer_rsrc_t rw0 =
      __builtin_amdgcn_make_buffer_rsrc((void*)wrow0, (short)0, wbytes0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw1 =
      __builtin_amdgcn_make_buffer_rsrc((void*)wrow1, (short)0, wbytes1, 0x00020000);
  const int kw = KMB ? ksplit / 64 : 0;   // K steps taken from W_g
  uint32_t woff[KMB ? NW : 4];
  int wput[NW];
  if constexpr (KMB) {
#pragma unroll
    for (int i = 0; i < NW; ++i) woff[i] = ((uint32_t)(8 * i + lr) * (uint32_t)N + (uint32_t)lc * 8u) * 2u;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) woff[q] = (uint32_t)(8 * q + lr) * (uint32_t)K * 2u + (uint32_t)lc * 16u;
  }
  const int warea = wave * WAREA;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int rw = 8 * i + lr;
    wput[i] = warea + rw * CH + (KMB ? (lc ^ (((rw >> 1) & 1) << 2)) : (lc ^ ((rw >> 1) & 7)));
  }
  // KMB fragment reads: byte offset of fragment j's first transposed read at
  // sub-step 0 (+ 1024 bytes per sub-step)
  uint32_t twb[2];
  {
    const int x = lane & 15, hq = (lane >> 4) & 1, sbit = (x >> 3) & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      twb[j] = (uint32_t)(warea * 16 + (32 * fh + (x >> 2)) * 128 +
                          (4 * (j ^ sbit) + 2 * hq + ((x & 3) >> 1)) * 16 + (x & 1) * 8);
  }
  // fragment reads: row 32 i + fr of a 32-row block, logical chunk 4 fh + s
  const int rsw = (fr >> 1) & 7;
  int cread[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) cread[s] = fr * CH + ((4 * fh + s) ^ rsw);

  u32x4 wr[4][NW];      // weight rows in flight, slot = K step % 4
  bf16x8 fw[2][2];      // weight fragments [sub-step parity][j]
  bf16x8 fa[2][MF];     // token fragments [sub-step parity][i]
  f32x16 acc[MF][2];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#define MOE_SB() __builtin_amdgcn_sched_barrier(0)
#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))
  // weight loads of K step kt into register slot sl (non-temporal: read once)
#define MOE_LW(kt, sl, i0, i1)                                                        \
  do {                                                                                \
    if constexpr (KMB) {                                                              \
      const int kq_ = (kt);                                                           \
      const bool hi_ = kq_ >= kw;                                                     \
      const int so_ = (hi_ ? kq_ - kw : kq_) * 128 * N;                               \
      _Pragma("unroll") for (int i_ = (i0); i_ < (i1); ++i_)                          \
        wr[sl][i_] = __builtin_amdgcn_raw_buffer_load_b128(hi_ ? rw1 : rw0, woff[i_], so_, 2); \
    } else {                                                                          \
      _Pragma("unroll") for (int i_ = (i0); i_ < (i1); ++i_)                          \
        wr[sl][i_] = __builtin_amdgcn_raw_buffer_load_b128(i_ < 4 ? rw0 : rw1, woff[i_ & 3], \
                                                           (kt) * 128, 2);           \
    }                                                                                 \
  } while (0)
  // token-row loads of K step kt into stage st (cached: the group's other slabs
  // read the same rows)
#define MOE_LA(kt, st)                                                                \
  do {                                                                                \
    _Pragma("unroll") for (int i_ = 0; i_ < NA; ++i_)                                 \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MOE_LDS(smem + ABASE + (st) * ASTAGE + (wave * MF + i_) * 64), \
                                               16, aoff[i_], (uint32_t)(kt) * 128u, 0, 0); \
  } while (0)
  // the weight rows of slot sl into this wave's LDS area
#define MOE_PUT(sl)                                                                   \
  do {                                                                                \
    _Pragma("unroll") for (int i_ = 0; i_ < NW; ++i_) smem[wput[i_]] = wr[sl][i_];    \
  } while (0)
#define MOE_RD(b, st, s)                                                              \
  do {                                                                                \
    if constexpr (KMB) {                                                              \
      fw[b][0] = lds_tr_frag<128>(smem, twb[0] + (s) * 1024);                         \
      fw[b][1] = lds_tr_frag<128>(smem, twb[1] + (s) * 1024);                         \
    } else {                                                                          \
      fw[b][0] = __builtin_bit_cast(bf16x8, smem[warea + cread[s]]);                  \
      fw[b][1] = __builtin_bit_cast(bf16x8, smem[warea + 32 * CH + cread[s]]);        \
    }                                                                                 \
    _Pragma("unroll") for (int i_ = 0; i_ < MF; ++i_)                                 \
      fa[b][i_] = __builtin_bit_cast(bf16x8, smem[ABASE + (st) * ASTAGE + i_ * 32 * CH + cread[s]]); \
  } while (0)
#define MOE_MM(b)                                                                     \
  do {                                                                                \
    _Pragma("unroll") for (int i_ = 0; i_ < MF; ++i_) {                               \
      acc[i_][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[b][0], fa[b][i_], acc[i_][0], 0, 0, 0); \
      acc[i_][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[b][1], fa[b][i_], acc[i_][1], 0, 0, 0); \
    }                                                                                 \
  } while (0)
  // K step kt (register slot and token stage sl = kt % 4; its weights already
  // in the wave's LDS area and its first fragments in fa[0] / fw[0]). LOAD
  // issues the loads of step kt + 3 (weights spread over the sub-steps, then
  // the token rows). Before the last sub-step's MFMAs: wait until the loads of
  // step kt + 1 have landed (vmcnt WAITN; all LDS reads of this step done),
  // barrier (publishes token stage kt + 1, retires stage kt), store the
  // weights of step kt + 1 into the wave's area and read the first fragments
  // of step kt + 1.
#define MOE_KSTEP(kt, sl, LOAD, WAITN, LAST)                                          \
  do {                                                                                \
    if (LOAD) MOE_LW((kt) + 3, ((sl) + 3) & 3, 0, 2);                                 \
    MOE_RD(1, sl, 1);                                                                 \
    MOE_SB();                                                                         \
    MOE_MM(0);                                                                        \
    MOE_SB();                                                                         \
    if (LOAD) MOE_LW((kt) + 3, ((sl) + 3) & 3, 2, 5);                                 \
    MOE_RD(0, sl, 2);                                                                 \
    MOE_SB();                                                                         \
    MOE_MM(1);                                                                        \
    MOE_SB();                                                                         \
    if (LOAD) MOE_LW((kt) + 3, ((sl) + 3) & 3, 5, 8);                                 \
    if (LOAD) MOE_LA((kt) + 3, ((sl) + 3) & 3);                                       \
    MOE_RD(1, sl, 3);                                                                 \
    MOE_SB();                                                                         \
    MOE_MM(0);                                                                        \
    MOE_SB();                                                                         \
    if (!(LAST)) {                                                                    \
      __builtin_amdgcn_s_waitcnt(stream_wait_imm(WAITN));                             \
      __builtin_amdgcn_s_barrier();                                                   \
      MOE_SB();                                                                       \
      MOE_PUT(((sl) + 1) & 3);                                                        \
      MOE_RD(0, ((sl) + 1) & 3, 0);                                                   \
      MOE_SB();                                                                       \
    }                                                                                 \
    MOE_MM(1);                                                                        \
    MOE_SB();                                                                         \
  } while (0)

  // prologue: steps 0, 1, 2 in flight (weights then token rows of each)
#pragma unroll
  for (int kt = 0; kt < 3; ++kt) {
    MOE_LW(kt, kt, 0, NW);
    MOE_LA(kt, kt);
  }
  __builtin_amdgcn_s_waitcnt(stream_wait_imm(2 * NL));
  __builtin_amdgcn_s_barrier();
  MOE_SB();
  MOE_PUT(0);
  MOE_RD(0, 0, 0);
  for (int kt = 0; kt < nk - 4; kt += 4) {
    MOE_KSTEP(kt + 0, 0, true, 2 * NL, false);
    MOE_KSTEP(kt + 1, 1, true, 2 * NL, false);
    MOE_KSTEP(kt + 2, 2, true, 2 * NL, false);
    MOE_KSTEP(kt + 3, 3, true, 2 * NL, false);
  }
  MOE_KSTEP(nk - 4, 0, true, 2 * NL, false);
  MOE_KSTEP(nk - 3, 1, false, NL, false);
  MOE_KSTEP(nk - 2, 2, false, 0, false);
  MOE_KSTEP(nk - 1, 3, false, 0, true);
#undef MOE_KSTEP
#undef MOE_MM
#undef MOE_RD
#undef MOE_PUT
#undef MOE_LA
#undef MOE_LW
#undef MOE_LDS
#undef MOE_SB

  // the block's count into the work queue's done counter, its round trip
  // under the epilogue's stores
  const int dn = threadIdx.x == 0 && done ? atomicAdd(done, 1) : -1;
  stream_epilogue<EPI, HAS_BIAS, MF>(acc, bg, row0, mrows, n0, C, N);
  return dn;
}

// The same tile on a packed copy of the weights (moe_pack_weights): per slab
// and K step, wave w's weight fragments are 8 KB in fragment order (fragment j,
// sub-step q, lane l: 16 bytes = row 32 j + l % 32 of the wave's 64 rows, K
// elements 32 (l / 32) + 8 q .. + 7 of the step), so each wave streams
// contiguous 1 KB runs from HBM straight into its MFMA operand registers,
// three K steps ahead, with no trip through LDS; only the token rows are
// staged in LDS (four stages, three ahead).
template <int EPI, bool HAS_BIAS, int MF>
__device__ __forceinline__ int stream_tile_packed(u32x4* __restrict__ smem,
                                                   const bf16* __restrict__ A, uint32_t a_bytes,
                                                   const int32_t* __restrict__ arows,
                                                   const bf16* __restrict__ Wpg, int slab,
                                                   const float* __restrict__ bg, int row0,
                                                   int mrows, int n0, bf16* __restrict__ C, int N,
                                                   int K, int* __restrict__ done) {
  constexpr int CH = 8;
  constexpr int ASTAGE = 32 * MF * CH;         // u32x4 per token-row stage
  constexpr int NW = 8, NA = MF, NL = NW + NA;
  static_assert(4 * ASTAGE <= kStreamLds, "LDS");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, fh = lane >> 5;
  const int nk = K / 64;                       // multiple of 4
  const int lr = lane >> 3, lc = lane & 7;

  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)a_bytes, 0x00020000);
  uint32_t aoff[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int rl = 8 * (wave * MF + i) + lr;
    const int r = row0 + min(rl, mrows - 1);
    const uint32_t rowoff = (uint32_t)(arows ? arows[r] : r) * (uint32_t)K * 2u;
    aoff[i] = rowoff + (uint32_t)(lc ^ ((rl >> 1) & 7)) * 16u;
  }
  // this wave's packed weights: 8 KB per K step, K steps 32 KB apart
  const char* wbase = reinterpret_cast<const char*>(Wpg) + ((int64_t)slab * nk * 4 + wave) * 8192;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)wbase, (short)0, (nk - 1) * 32768 + 8192, 0x00020000);
  const uint32_t wlane = (uint32_t)lane * 16u;
  const int rsw = (fr >> 1) & 7;
  int cread[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) cread[s4] = fr * CH + ((4 * fh + s4) ^ rsw);

  bf16x8 wr[4][2][4];   // weight fragments in flight [slot = K step % 4][j][sub-step]
  bf16x8 fa[MF];        // token fragments of the current sub-step
  f32x16 acc[MF][2];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#define MOE_SB() __builtin_amdgcn_sched_barrier(0)
#define MOE_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define MOE_LW(kt, sl, q)                                                             \
  do {                                                                                \
    wr[sl][0][q] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(  \
                                                 rw, wlane + (q) * 1024u, (kt) * 32768, 2)); \
    wr[sl][1][q] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(  \
                                                 rw, wlane + (4 + (q)) * 1024u, (kt) * 32768, 2)); \
  } while (0)
#define MOE_LA(kt, st)                                                                \
  do {                                                                                \
    _Pragma("unroll") for (int i_ = 0; i_ < NA; ++i_)                                 \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MOE_LDS(smem + (st) * ASTAGE + (wave * MF + i_) * 64), \
                                               16, aoff[i_], (uint32_t)(kt) * 128u, 0, 0); \
  } while (0)
  // Sub-step s of the step in slot sl: for each token fragment i, its two
  // MFMAs and the read of fragment i for (stage srd, sub-step s2) into the same
  // registers (the compiler interleaves these freely: fixing the order pair by
  // pair with scheduling barriers cost 1.5-2.5 % of the GEMM stages); then
  // (LOAD) the weight loads of step kl, sub-step s, into slot (sl + 3) & 3, the
  // previous step's slot, behind a scheduling barrier so that the order of the
  // loads, which the vmcnt waits count, stays fixed.
#define MOE_SUB(sl, s, srd, s2, LOAD, kl)                                             \
  do {                                                                                \
    _Pragma("unroll") for (int i_ = 0; i_ < MF; ++i_) {                               \
      acc[i_][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[sl][0][s], fa[i_], acc[i_][0], 0, 0, 0); \
      acc[i_][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[sl][1][s], fa[i_], acc[i_][1], 0, 0, 0); \
      fa[i_] = __builtin_bit_cast(bf16x8, smem[(srd) * ASTAGE + i_ * 32 * CH + cread[s2]]); \
    }                                                                                 \
    if (LOAD) MOE_LW(kl, ((sl) + 3) & 3, s);                                          \
    MOE_SB();                                                                         \
  } while (0)
  // K step kt (register slot and token stage sl = kt % 4). Issue order per
  // step: weights of step kt + 3 for sub-steps 0..2, its token rows, then (after
  // the barrier) its weights for sub-step 3. Before the last sub-step: wait
  // until the token rows of step kt + 1 have landed (vmcnt WAITN) and all LDS
  // reads of this step are done, barrier; the last sub-step then reads the
  // first token fragments of step kt + 1.
#define MOE_KSTEP(kt, sl, LOAD, WAITN, LAST)                                          \
  do {                                                                                \
    MOE_SUB(sl, 0, sl, 1, LOAD, (kt) + 3);                                            \
    MOE_SUB(sl, 1, sl, 2, LOAD, (kt) + 3);                                            \
    MOE_SUB(sl, 2, sl, 3, LOAD, (kt) + 3);                                            \
    if (LOAD) MOE_LA((kt) + 3, ((sl) + 3) & 3);                                       \
    if (!(LAST)) {                                                                    \
      __builtin_amdgcn_s_waitcnt(stream_wait_imm(WAITN));                             \
      __builtin_amdgcn_s_barrier();                                                   \
      MOE_SB();                                                                       \
      MOE_SUB(sl, 3, ((sl) + 1) & 3, 0, LOAD, (kt) + 3);                              \
    } else {                                                                          \
      _Pragma("unroll") for (int i_ = 0; i_ < MF; ++i_) {                             \
        acc[i_][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[sl][0][3], fa[i_], acc[i_][0], 0, 0, 0); \
        acc[i_][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[sl][1][3], fa[i_], acc[i_][1], 0, 0, 0); \
      }                                                                               \
    }                                                                                 \
  } while (0)

  // prologue: steps 0, 1, 2 in the steady-state issue order (sub-steps 0..2,
  // token rows, sub-step 3); wait for the token rows of step 0
#pragma unroll
  for (int kt = 0; kt < 3; ++kt) {
#pragma unroll
    for (int q = 0; q < 3; ++q) MOE_LW(kt, kt, q);
    MOE_LA(kt, kt);
    MOE_LW(kt, kt, 3);
  }
  __builtin_amdgcn_s_waitcnt(stream_wait_imm(2 * NL + 2));
  __builtin_amdgcn_s_barrier();
  MOE_SB();
#pragma unroll
  for (int i = 0; i < MF; ++i) fa[i] = __builtin_bit_cast(bf16x8, smem[i * 32 * CH + cread[0]]);
  MOE_SB();
  // loads issued after the token rows of step kt + 1, at the wait of step kt:
  // steady state 2 NL; then NL + 2 and 2 for the last two waits
  for (int kt = 0; kt < nk - 4; kt += 4) {
    MOE_KSTEP(kt + 0, 0, true, 2 * NL, false);
    MOE_KSTEP(kt + 1, 1, true, 2 * NL, false);
    MOE_KSTEP(kt + 2, 2, true, 2 * NL, false);
    MOE_KSTEP(kt + 3, 3, true, 2 * NL, false);
  }
  MOE_KSTEP(nk - 4, 0, true, 2 * NL, false);
  MOE_KSTEP(nk - 3, 1, false, NL + 2, false);
  MOE_KSTEP(nk - 2, 2, false, 2, false);
  MOE_KSTEP(nk - 1, 3, false, 0, true);
#undef MOE_KSTEP
#undef MOE_SUB
#undef MOE_LA
#undef MOE_LW
#undef MOE_LDS
#undef MOE_SB
  // the block's count into the work queue's done counter, its round trip
  // under the epilogue's stores
  const int dn = threadIdx.x == 0 && done ? atomicAdd(done, 1) : -1;
  stream_epilogue_lds<EPI, HAS_BIAS, MF>(acc, smem, bg, row0, mrows, n0, C, N);
  return dn;
}

// Work item t of the streaming GEMM (group, rows, slab from the item space ss):
// one tile. Returns the block's count into the done counter (thread 0; -1
// without one).
// KMB: K-major weights as stream_tile's KMB (W_g = W + g ksplit N, W3_g =
// W3 + g (K - ksplit) N; the shared expert Ws / Ws3), standard layout only.
template <int EPI, bool HAS_BIAS, bool KMB = false>
__device__ __forceinline__ int stream_item(u32x4* __restrict__ smem, const StreamSpace& ss, int t,
                                           int ns, const bf16* __restrict__ A,
                                           const bf16* __restrict__ W, const bf16* __restrict__ W3,
                                           const float* __restrict__ bias,
                                           const bf16* __restrict__ Ws, const bf16* __restrict__ Ws3,
                                           const float* __restrict__ bias_s, int E,
                                           bf16* __restrict__ C, int N, int K,
                                           const int32_t* __restrict__ arows, uint32_t a_bytes,
                                           const bf16* __restrict__ Wp, int* __restrict__ done,
                                           int ksplit = 0) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  constexpr int BNO = GATED ? 128 : 256;
  int g, row0, nrows, slab;
  stream_lookup(ss, t, ns, g, row0, nrows, slab);
  g = __builtin_amdgcn_readfirstlane(g);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  nrows = __builtin_amdgcn_readfirstlane(nrows);
  slab = __builtin_amdgcn_readfirstlane(slab);
  const int n0 = slab * BNO;
  if constexpr (KMB) {
    const bf16* Wk = g < E ? W + (int64_t)g * ksplit * N : Ws;
    const bf16* W3k = W3 ? (g < E ? W3 + (int64_t)g * (K - ksplit) * N : Ws3) : nullptr;
    const int mfk = (nrows + 31) / 32;
    if (mfk <= 2)
      return stream_tile<EPI, HAS_BIAS, 2, true>(smem, A, a_bytes, arows, Wk, W3k, nullptr, row0,
                                                 nrows, n0, C, N, K, done, ksplit);
    if (mfk <= 4)
      return stream_tile<EPI, HAS_BIAS, 4, true>(smem, A, a_bytes, arows, Wk, W3k, nullptr, row0,
                                                 nrows, n0, C, N, K, done, ksplit);
    if (mfk <= 6)
      return stream_tile<EPI, HAS_BIAS, 6, true>(smem, A, a_bytes, arows, Wk, W3k, nullptr, row0,
                                                 nrows, n0, C, N, K, done, ksplit);
    return stream_tile<EPI, HAS_BIAS, 8, true>(smem, A, a_bytes, arows, Wk, W3k, nullptr, row0,
                                               nrows, n0, C, N, K, done, ksplit);
  } else {
  const bf16* Wg = g < E ? W + (int64_t)g * N * K : Ws;
  const bf16* W3g = GATED ? (g < E ? W3 + (int64_t)g * N * K : Ws3) : Wg;
  const float* bg = HAS_BIAS ? (g < E ? bias + (int64_t)g * N : bias_s) : nullptr;
  const int mf = (nrows + 31) / 32;
  // packed weights of group g: (SwiGLU: 2 x) N x K elements per group; with
  // them, rows rounded up to the next multiple of 32 (MF = 1 .. 8 fragments)
  const bf16* Wpg = Wp ? Wp + (int64_t)g * (GATED ? 2 : 1) * N * K : nullptr;
  int dn;   // this block's count into the done counter (thread 0)
  if (Wp) {
#define MOE_PT(M)                                                                     \
  stream_tile_packed<EPI, HAS_BIAS, M>(smem, A, a_bytes, arows, Wpg, slab, bg, row0, nrows, n0, C, N, K, \
                                       done)
    switch (mf) {
      case 1: dn = MOE_PT(1); break;
      case 2: dn = MOE_PT(2); break;
      case 3: dn = MOE_PT(3); break;
      case 4: dn = MOE_PT(4); break;
      case 5: dn = MOE_PT(5); break;
      case 6: dn = MOE_PT(6); break;
      case 7: dn = MOE_PT(7); break;
      default: dn = MOE_PT(8); break;
    }
#undef MOE_PT
  } else if (mf <= 2) {
    dn = stream_tile<EPI, HAS_BIAS, 2>(smem, A, a_bytes, arows, Wg, W3g, bg, row0, nrows, n0, C, N, K, done);
  } else if (mf <= 4) {
    dn = stream_tile<EPI, HAS_BIAS, 4>(smem, A, a_bytes, arows, Wg, W3g, bg, row0, nrows, n0, C, N, K, done);
  } else if (mf <= 6) {
    dn = stream_tile<EPI, HAS_BIAS, 6>(smem, A, a_bytes, arows, Wg, W3g, bg, row0, nrows, n0, C, N, K, done);
  } else {
    dn = stream_tile<EPI, HAS_BIAS, 8>(smem, A, a_bytes, arows, Wg, W3g, bg, row0, nrows, n0, C, N, K, done);
  }
  return dn;
  }
}

// Work-queue counters of the streaming GEMM: kSchedSlots slots per device of
// 9 counters (the 8 per-XCD ticket counters, then the count of blocks done
// with the queue), each in a 64-byte line of its own (kSchedStride ints
// apart) so that atomics on different counters do not queue behind each
// other; zero when the library is loaded and put back to zero by the last
// block of each launch. Launches take the slots in turn, so launches in
// flight at the same time (on other streams) use different slots as long as
// fewer than kSchedSlots of them overlap.
constexpr int kSchedSlots = 256;
constexpr int kSchedStride = 16;
constexpr int kSchedSlotInts = 16 * kSchedStride;
__device__ int g_stream_sched[kSchedSlots * kSchedSlotInts];

// One launch over every group with rows in (0, max_rows] ((min_last, max_last]
// for the last group). The work items (group, slab, part) in group order are split
// into 8 ranges of equal count, one per XCD. A block takes a ticket of its own
// XCD's range: the range's counter hands out its items in reverse order, so
// that the last range starts with the last group (the shared expert's items,
// the heaviest). A block whose range is used up reads the other ranges'
// counters and takes a ticket of one that still has items, until it gets an
// item or reads every range used up (then it exits). The grid has at least as
// many blocks as items, so every item is taken: a block leaves without one
// only after reading every counter at its range's size. Items of one group,
// and the parts of one slab, thus mostly run at the same time on one XCD and
// share its L2, while a range whose items are heavier than the others' is
// finished by the blocks of the other XCDs.
// The counters are those of the slot at sched, zero on entry; every block adds
// one to the done counter after its last ticket (a working block at the start
// of its epilogue), and the block that adds the last puts them back to zero.
// In a launch with no items every block gives its ticket back instead.
// With sched null the order is static: block b takes item (b % 8) n / 8 +
// b / 8 of the n items (blocks are dispatched to the XCDs round-robin), and
// blocks past the item count exit.
// Requires N a multiple of 256, K a multiple of 256, and the A operand
// addressable with 32-bit byte offsets (a_bytes < 2^32; checked by the host).
// KMB: the weights K-major as stored (stream_item's KMB; ksplit as there).
template <int EPI, bool HAS_BIAS, bool KMB = false>
__global__ __launch_bounds__(256, 1) void gemm_stream_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* __restrict__ W3,
    const float* __restrict__ bias, const bf16* __restrict__ Ws, const bf16* __restrict__ Ws3,
    const float* __restrict__ bias_s, int E, int G, const int32_t* __restrict__ offsets,
    int rows_max, bf16* __restrict__ C, int N, int K, const int32_t* __restrict__ arows,
    uint32_t a_bytes, int max_rows, int min_last, int max_last, const bf16* __restrict__ Wp,
    int* __restrict__ sched, int ksplit) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  constexpr int BNO = GATED ? 128 : 256;   // output columns per slab
  __shared__ u32x4 smem[kStreamLds];   // the K-step stages (160 KB, all of the CU's LDS)
  const int ns = N / BNO;
  StreamSpace ss;
  int t;
  if (!sched) {
    // static order: block b takes item b of the XCD-aware order (blocks are
    // dispatched to the XCDs round-robin, and XCD b % 8 runs range b % 8 of
    // the items, in order); blocks past the item count exit
    stream_space_init(ss, offsets, G, rows_max, max_rows, min_last, max_last, ns);
    const int items = __builtin_amdgcn_readfirstlane(ss.total);
    const int b = blockIdx.x;
    if (b >= items) return;
    const int t8 = items & ~7;
    t = b < t8 ? (b & 7) * (t8 >> 3) + (b >> 3) : b;
  } else {
    // a ticket of this block's XCD range first (hardware register XCC_ID); its
    // round trip overlaps the offsets' loads
    int xcc = 0, tk = 0;
    if (threadIdx.x == 0) {
      xcc = (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7u);
      tk = atomicAdd(&sched[xcc * kSchedStride], 1);
    }
    stream_space_init(ss, offsets, G, rows_max, max_rows, min_last, max_last, ns);
    const int items = __builtin_amdgcn_readfirstlane(ss.total);
    if (items == 0) {
      // nothing to do in this launch (every block sees the same offsets): give
      // the ticket back, so the counters end at zero without the done count
      if (threadIdx.x == 0) atomicSub(&sched[xcc * kSchedStride], 1);
      return;
    }
    if (threadIdx.x == 0) {
      auto lo_of = [&](int x) { return (int)((int64_t)items * x / 8); };
      int item = -1;
      if (tk < lo_of(xcc + 1) - lo_of(xcc)) {
        item = lo_of(xcc + 1) - 1 - tk;
      } else {
        // own range used up: read all eight counters (one round trip), take a
        // ticket of the first other range that still has items, and read again
        // if someone was quicker; a block that reads every range used up exits
        for (;;) {
          int c[8];
#pragma unroll
          for (int x = 0; x < 8; ++x)
            c[x] = __hip_atomic_load(&sched[x * kSchedStride], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          int pick = -1;
#pragma unroll
          for (int q = 1; q < 8; ++q) {
            const int x = (xcc + q) & 7;
            if (pick < 0 && c[x] < lo_of(x + 1) - lo_of(x)) pick = x;
          }
          if (pick < 0) break;
          const int tq = atomicAdd(&sched[pick * kSchedStride], 1);
          if (tq < lo_of(pick + 1) - lo_of(pick)) {
            item = lo_of(pick + 1) - 1 - tq;
            break;
          }
        }
      }
      reinterpret_cast<int*>(smem)[0] = item;   // broadcast through LDS
      if (item < 0) {
        // no item: done with the queue now
        __threadfence();
        if (atomicAdd(&sched[8 * kSchedStride], 1) == (int)gridDim.x - 1)
          for (int x = 0; x < 9; ++x) atomicExch(&sched[x * kSchedStride], 0);
      }
    }
    __syncthreads();
    t = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(smem)[0]);
    __syncthreads();   // read by every wave before the tile's loads land in LDS
    if (t < 0) return;
  }
  const int dn = stream_item<EPI, HAS_BIAS, KMB>(smem, ss, t, ns, A, W, W3, bias, Ws, Ws3, bias_s,
                                                 E, C, N, K, arows, a_bytes, Wp,
                                                 sched ? sched + 8 * kSchedStride : nullptr, ksplit);
  if (sched && threadIdx.x == 0 && dn == (int)gridDim.x - 1)
    for (int x = 0; x < 9; ++x) atomicExch(&sched[x * kSchedStride], 0);
}

// float32 layers: one thread per (row, column) of a tile, plain FMA loop.
template <int EPI, bool HAS_BIAS>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ W, const float* __restrict__ W3,
    const float* __restrict__ bias, const float* __restrict__ Ws, const float* __restrict__ Ws3,
    const float* __restrict__ bias_s, int E, int G, const int32_t* __restrict__ offsets,
    int rows_max, float* __restrict__ C, int N, int K, const int32_t* __restrict__ arows) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  const int ncb = (N + 255) / 256;
  const int mt = blockIdx.x / ncb;
  const int n = (blockIdx.x - mt * ncb) * 256 + threadIdx.x;
  int g, row0, nrows;
  if (!find_tile(offsets, G, rows_max, kGemmBM, mt, g, row0, nrows)) return;
  if (n >= N) return;
  const float* w = (g < E ? W + (int64_t)g * N * K : Ws) + (int64_t)n * K;
  const float* w3 = GATED ? (g < E ? W3 + (int64_t)g * N * K : Ws3) + (int64_t)n * K : nullptr;
  const float bv = HAS_BIAS ? (g < E ? bias + (int64_t)g * N : bias_s)[n] : 0.f;
  for (int m = 0; m < nrows; ++m) {
    const float* a = A + (int64_t)(arows ? arows[row0 + m] : row0 + m) * K;
    float s1 = 0.f, s3 = 0.f;
    for (int kk = 0; kk < K; ++kk) {
      s1 = fmaf(a[kk], w[kk], s1);
      if (GATED) s3 = fmaf(a[kk], w3[kk], s3);
    }
    C[(int64_t)(row0 + m) * N + n] = epilogue<EPI>(s1 + bv, s3);
  }
}

// Packed copy of a group's weights in the order the streaming GEMM's packed
// tile reads them. 16-byte unit u of group g: lane l = u % 64, sub-step
// q = (u / 64) % 4, fragment j = (u / 256) % 2, wave w = (u / 512) % 4, K step
// k and slab s from u / 2048; it holds K elements 64 k + 32 (l / 32) + 8 q ..
// + 7 of weight row (SwiGLU: j = 0 row 128 s + 32 w + l % 32 of W1, j = 1 the
// same row of W3; otherwise row 256 s + 64 w + 32 j + l % 32 of W). Groups
// g < E come from W (W3) + g N K, group E from Ws (Ws3).
template <bool GATED>
__global__ __launch_bounds__(256) void pack_weights_kernel(
    const bf16* __restrict__ W, const bf16* __restrict__ W3, const bf16* __restrict__ Ws,
    const bf16* __restrict__ Ws3, int E, int G, int N, int K, u32x4* __restrict__ out) {
  const int nk = K / 64;
  const int64_t per_group = (int64_t)(GATED ? 2 : 1) * N * K / 8;   // 16-byte units
  const int64_t total = per_group * G;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total; u += (int64_t)gridDim.x * 256) {
    const int g = (int)(u / per_group);
    const int64_t v = u - (int64_t)g * per_group;
    const int l = (int)(v & 63), q = (int)((v >> 6) & 3), j = (int)((v >> 8) & 1),
              w = (int)((v >> 9) & 3);
    const int64_t rest = v >> 11;
    const int k = (int)(rest % nk);
    const int s = (int)(rest / nk);
    const bf16* src;
    int row;
    if (GATED) {
      src = j == 0 ? (g < E ? W + (int64_t)g * N * K : Ws) : (g < E ? W3 + (int64_t)g * N * K : Ws3);
      row = 128 * s + 32 * w + (l & 31);
    } else {
      src = g < E ? W + (int64_t)g * N * K : Ws;
      row = 256 * s + 64 * w + 32 * j + (l & 31);
    }
    out[u] = *reinterpret_cast<const u32x4*>(src + (int64_t)row * K + 64 * k + 32 * (l >> 5) + 8 * q);
  }
}

// Device address of this launch's slot of g_stream_sched (slots taken in turn;
// the array's address resolved once per device), or nullptr on failure.
static int* stream_sched_slot() {
  static std::mutex mu;
  static int* base[64] = {nullptr};
  static std::atomic<unsigned> next{0};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!base[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_stream_sched)) != hipSuccess || !p) return nullptr;
      base[dev] = static_cast<int*>(p);
    }
  }
  return base[dev] + (next.fetch_add(1) % kSchedSlots) * kSchedSlotInts;
}

// Block slots of the persistent 128 x 128 kernel on the current device: two
// per CU, a multiple of 8 (one share per XCD), cached per device.
// Left-over rows of the tiled path (tile space part 2: each group's rows past
// its full 256-row tiles) split along K: kparts float32 planes of the rest
// tiles, [kparts][cap 128][N] by M tile, written by gemm_bf16_kernel<EPI_PARTIAL>
// and added here in plane order, then the bias and the rounding:
// C[row0 + m][n] = bf16(sum_kp P[kp][128 mt + m][n] + b_g[n]). Block: M tile
// blockIdx.x, 4 of its rows (blockIdx.y), 8 columns per thread, the planes'
// loads issued together.
template <bool HAS_BIAS>
__global__ __launch_bounds__(256) void rest_reduce_kernel(
    const float* __restrict__ P, int kparts, int cap, const int32_t* __restrict__ offsets, int G,
    int E, int rows_max, int skip_rows, int skip_last, const float* __restrict__ bias,
    const float* __restrict__ bias_s, int N, bf16* __restrict__ C) {
  TileSpace ts;
  tile_space_init(ts, offsets, G, rows_max, 128, 2, kGemmBigBM, skip_rows, skip_last);
  const int mt = blockIdx.x;
  if (mt >= ts.total || mt >= cap) return;
  int g, row0, nrows;
  tile_lookup(ts, mt, 128, g, row0, nrows);
  const float* bg = HAS_BIAS ? (g < E ? bias + (int64_t)g * N : bias_s) : nullptr;
  const int c8 = N / 8;
  const int64_t plane = (int64_t)cap * 128 * N;
  for (int idx = threadIdx.x; idx < 4 * c8; idx += 256) {
    const int m = blockIdx.y * 4 + idx / c8;
    const int c = (idx % c8) * 8;
    if (m >= nrows) continue;
    const float* p0 = P + ((int64_t)mt * 128 + m) * N + c;
    float v[8], w[3][8];
    load8(p0, v);
#pragma unroll
    for (int q = 0; q < 3; ++q) {   // planes 1..3 (kparts <= 4)
      if (q + 1 < kparts) {
        load8(p0 + (q + 1) * plane, w[q]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[q][e] = 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (q + 1 < kparts) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += w[q][e];
      }
    if (HAS_BIAS) {
      float b[8];
      load8(bg + c, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += b[e];
    }
    store8(C + (int64_t)(row0 + m) * N + c, v);
  }
}

// Plan of that split for a GEMM of N columns and K depth whose groups of at
// most skip rows are streamed (skip 0: none): the rest tiles number at most
// cap = 2 per group on the tiled path (groups of more than skip rows, at most
// rows_max / (skip + 1) of them); split into kparts = 4 (2) ranges of at least
// 4 K steps when they would otherwise fill under a quarter of the CU slots
// (at most 256 tiles) and their planes fit 64 MiB. kparts 1: no split.
RestSplit rest_split_plan(const moe_config& c, int N, int K, int skip) {
  RestSplit r{1, 0, 0};
  if (c.act_dtype != MOE_BF16 || N % 128 || K % 64) return r;
  const int64_t G = c.num_experts + c.num_shared_experts;
  const int64_t rows = rows_max(c);
  int64_t cap = 2 * G;
  if (skip > 0) cap = std::min<int64_t>(cap, 2 * (rows / (skip + 1)) + 2);
  if (cap <= 0 || cap * (N / 128) > 256) return r;
  const int nk = K / 64;
  const int kp = nk % 8 == 0 && nk / 4 >= 4 ? 4 : (nk % 4 == 0 && nk / 2 >= 4 ? 2 : 1);
  const size_t bytes = (size_t)kp * cap * 128 * N * 4;
  if (kp == 1 || bytes > ((size_t)64 << 20)) return r;
  r.kparts = kp;
  r.cap = (int)cap;
  r.bytes = bytes;
  return r;
}

static int gemm_slots() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = (2 * cus) & ~7 ? (2 * cus) & ~7 : 8;
  }
  return cached[dev];
}

// KMB: bf16 weights read K-major as stored ([K][N] per group, W3 / Ws3 for K
// steps from ksplit on; backward dZ and dX): groups of at most kStreamMaxRows
// rows on the weight-streaming kernel where the epilogue is linear, the rest
// on the tiled kernels.
template <typename ET, int EPI, bool HB, bool KMB = false>
static hipError_t gemm_launch(const moe_config& c, const ET* A, const void* W, const void* W3,
                              const float* bias, const void* Ws, const void* Ws3,
                              const float* bias_s, const int32_t* offsets, ET* C, int N, int K,
                              hipStream_t s, const int32_t* arows = nullptr,
                              const bf16* zin = nullptr, const void* wpacked = nullptr,
                              int ksplit = 0, float* colsum = nullptr, int colsum_tiles = 0,
                              float* rest_partial = nullptr, size_t rest_bytes = 0) {
  static_assert(!KMB || sizeof(ET) == 2, "K-major weights: bf16 only");
  const int E = c.num_experts, G = c.num_experts + c.num_shared_experts;
  const int64_t rows = rows_max(c);
  if constexpr (sizeof(ET) == 2) {
    constexpr int BNB = EPI == EPI_SWIGLU ? 128 : 256;
    constexpr int BN = EPI == EPI_SWIGLU ? 64 : 128;
    // the 128 x 128 kernel is persistent: at most two blocks per CU, each
    // looping over the tiles (grid bounds below; surplus blocks exit)
    const int slots = gemm_slots();
    // 256 x 256 tiles pay off for the GEMMs without an activation whose
    // output is at most 4096 wide (the DeepSpeed-GPT shape's GEMM 2: 256 tiles,
    // one per CU): with an activation, one block per CU leaves the epilogue's
    // VALU work exposed, which two 128 x 128 blocks per CU hide behind each
    // other's MFMAs; and at N = 7168 or a long K (the DeepSeek-V3 shared expert)
    // the 128 x 128 kernel's two K steps in flight and finer tail were faster
    // (one MI355X: 2.60 -> 2.56 ms GEMM 1, 1.53 -> 1.50 ms GEMM 2 stages).
    // gathered A rows (arows) are addressed with 32-bit offsets from the start
    // of x, which the 256 x 256 kernel's buffer loads need below 4 GiB
    const int64_t a_bytes = arows ? c.tokens * (int64_t)K * 2 : 0;
    // Groups of at most kStreamMaxRows rows go to the weight-streaming kernel
    // (forward epilogues; its A operand addressed with 32-bit byte offsets),
    // the others to the 256 x 256 and 128 x 128 kernels below.
    // (K-major weights, the backward's dH and dX: the linear epilogue only)
    constexpr bool kStreamEpi = KMB ? EPI == EPI_NONE
                                    : (EPI == EPI_GELU || EPI == EPI_RELU || EPI == EPI_SWIGLU ||
                                       EPI == EPI_NONE);
    const int64_t a_span = arows ? a_bytes : rows * (int64_t)K * 2;
    // (K-major: the streaming tile addresses a group's weights, K x N bf16, with
    // 32-bit signed byte counts)
    const bool kmb_fits = !KMB || (int64_t)K * N * 2 < ((int64_t)1 << 31);
    const int skip = kStreamEpi && kmb_fits && a_span < ((int64_t)1 << 32) ? kStreamMaxRows : 0;
    // a shared expert (the last group, nominally T rows) of up to
    // kStreamSharedMaxRows rows is streamed too (at the DeepSeek-V3 shape,
    // T = 4096 and K = 7168, faster than on the tiled kernels)
    const int skip_last =
        skip > 0 && G > E && c.tokens > skip && c.tokens <= kStreamSharedMaxRows ? kStreamSharedMaxRows
                                                                                  : skip;
    if constexpr (kStreamEpi) {
      if (skip > 0) {
        constexpr int BNO = EPI == EPI_SWIGLU ? 128 : 256;
        // items: parts x N / BNO slabs, where the parts, ceil(r_g / 256) summed
        // over the groups taken (r_g in (0, skip]), are at most
        // (rows + 255 G) / 256 and at most ceil(skip / 256) G
        // The work queue (see gemm_stream_kernel) where the routed groups
        // average 512 to 1536 rows (several parts per slab: the Mixtral shape,
        // both GEMM stages 4-6 % faster, paired timing on one MI355X); the
        // static order for fine-grained experts (the DeepSeek-V3 shape, whose
        // many short items pay more for the queue's atomics than its balance
        // gains: GEMM 2 stage 2-4 % slower with it), and where the groups are
        // expected to be too large for this kernel (an empty launch is cheaper
        // without tickets).
        int* sched = nullptr;
        const int64_t assigned = (int64_t)c.top_k * c.tokens;
        if (assigned >= (int64_t)512 * E && assigned <= (int64_t)skip * E) {
          sched = stream_sched_slot();
          if (!sched) return hipErrorInvalidSymbol;
        }
        const int64_t parts = std::min<int64_t>((rows + (int64_t)(kStreamRows - 1) * G) / kStreamRows,
                                                (int64_t)G * ((skip + kStreamRows - 1) / kStreamRows));
        const int64_t items = parts * (N / BNO);
        if (items > 0)
          hipLaunchKernelGGL((gemm_stream_kernel<EPI, HB, KMB>), dim3((unsigned)items), dim3(256), 0,
                             s, A, (const bf16*)W, (const bf16*)W3, bias, (const bf16*)Ws,
                             (const bf16*)Ws3, bias_s, E, G, offsets, (int)rows, C, N, K, arows,
                             (uint32_t)a_span, skip, 0, skip, (const bf16*)wpacked, sched, ksplit);
        // The shared expert (group E, nominally T rows) with more than skip and
        // at most skip_last rows: a launch of its own over group E alone (at
        // most 16 parts of 256 rows per slab), in place of the tiled kernels
        // (at the DeepSeek-V3 shape, T = 4096 and K = 7168: GEMM 1 stage
        // 2.76 -> 2.69 ms, paired timing on one MI355X). Separate rather than
        // in the launch above: there the heavy shared items made GEMM 2 slower.
        if (skip_last > skip) {
          int* sched2 = nullptr;
          if (sched) {
            sched2 = stream_sched_slot();
            if (!sched2) return hipErrorInvalidSymbol;
          }
          const size_t per_group = (size_t)(EPI == EPI_SWIGLU ? 2 : 1) * N * K;
          hipLaunchKernelGGL((gemm_stream_kernel<EPI, HB, KMB>),
                             dim3((unsigned)(kStreamSharedMaxRows / kStreamRows * (N / BNO))),
                             dim3(256), 0, s, A, (const bf16*)W, (const bf16*)W3, bias,
                             (const bf16*)Ws, (const bf16*)Ws3, bias_s, 0, 1, offsets + E,
                             (int)rows, C, N, K, arows, (uint32_t)a_span, skip, skip, skip_last,
                             wpacked ? (const bf16*)wpacked + (size_t)E * per_group : nullptr,
                             sched2, ksplit);
        }
      }
    }
    // (the backward epilogues EPI_DGELU / EPI_DRELU exist in the 128 x 128 kernel only)
    const bool big = rows >= kGemmBigBM && EPI == EPI_NONE && N <= 4096 &&
                     EPI != EPI_DGELU && EPI != EPI_DRELU && a_bytes < ((int64_t)1 << 32);
    if (big) {
      // full 256-row tiles of each group, then the rows left over (< 256 per
      // group) in 128-row tiles; both grids are bounds, surplus blocks exit
      const unsigned big_tiles = (unsigned)(rows / kGemmBigBM) * (unsigned)(N / BNB);
      if constexpr (EPI != EPI_DGELU && EPI != EPI_DRELU)
        hipLaunchKernelGGL((gemm_bf16_big_kernel<EPI, HB, KMB>), dim3(big_tiles), dim3(256), 0, s, A,
                           (const bf16*)W, (const bf16*)W3, bias, (const bf16*)Ws, (const bf16*)Ws3,
                           bias_s, E, G, offsets, (int)rows, C, N, K, arows, (uint32_t)a_bytes,
                           skip, skip_last, ksplit);
      // each group leaves at most 255 rows, i.e. at most 2 tiles, and the
      // tiles number at most ceil(rows / 128) + G
      const int64_t rest = (rows + 127) / 128 + G < 2 * G ? (rows + 127) / 128 + G : 2 * G;
      const RestSplit rs = rest_partial ? rest_split_plan(c, N, K, skip) : RestSplit{1, 0, 0};
      if (rs.kparts > 1 && rs.bytes <= rest_bytes) {
        // few left-over tiles with a long K (the DeepSpeed-GPT shape's GEMM 2
        // and dX): split along K into float32 planes, then add them
        const int64_t items = (int64_t)rs.cap * (N / 128) * rs.kparts;
        hipLaunchKernelGGL((gemm_bf16_kernel<EPI_PARTIAL, false, KMB>),
                           dim3((unsigned)(items < slots ? items : slots)), dim3(256), 0, s, A,
                           (const bf16*)W, (const bf16*)W3, (const float*)nullptr, (const bf16*)Ws,
                           (const bf16*)Ws3, (const float*)nullptr, E, G, offsets, (int)rows,
                           (void*)rest_partial, N, K, 2, arows, rs.kparts, (const bf16*)nullptr,
                           skip, skip_last, ksplit, (float*)nullptr, rs.cap);
        hipLaunchKernelGGL((rest_reduce_kernel<HB>), dim3((unsigned)rs.cap, 32), dim3(256), 0, s,
                           (const float*)rest_partial, rs.kparts, rs.cap, offsets, G, E, (int)rows,
                           skip, skip_last, bias, bias_s, N, (bf16*)C);
      } else {
        const int64_t rgrid = rest * (N / BN) < slots ? rest * (N / BN) : slots;
        hipLaunchKernelGGL((gemm_bf16_kernel<EPI, HB, KMB>), dim3((unsigned)rgrid), dim3(256), 0, s, A,
                           (const bf16*)W, (const bf16*)W3, bias, (const bf16*)Ws, (const bf16*)Ws3,
                           bias_s, E, G, offsets, (int)rows, C, N, K, 2, arows, 1, zin, skip,
                           skip_last, ksplit, (float*)nullptr, 0);
      }
    } else {
      const int64_t tiles = ((rows + 127) / 128 + G) * (N / BN);
      const int64_t grid = tiles < slots ? tiles : slots;
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI, HB, KMB>), dim3((unsigned)grid), dim3(256), 0, s, A,
                         (const bf16*)W, (const bf16*)W3, bias, (const bf16*)Ws, (const bf16*)Ws3,
                         bias_s, E, G, offsets, (int)rows, C, N, K, 0, arows, 1, zin, skip,
                         skip_last, ksplit, colsum, colsum_tiles);
    }
  } else {
    const unsigned mtiles = (unsigned)((rows + kGemmBM - 1) / kGemmBM) + G;
    hipLaunchKernelGGL((gemm_f32_kernel<EPI, HB>), dim3(mtiles * ((N + 255) / 256)), dim3(256), 0,
                       s, A, (const float*)W, (const float*)W3, bias, (const float*)Ws,
                       (const float*)Ws3, bias_s, E, G, offsets, (int)rows, C, N, K, arows);
  }
  return hipGetLastError();
}

// Router logits on MFMA where both x and W_g are bf16 and E is a multiple of
// 128 (the 128-expert and 256-expert layers, whose gate GEMM is 2-15 GFLOP):
// the 128 x 128 kernel runs over the single group of T rows with its K loop
// cut into kparts ranges (one 128-row tile x 128 experts per work item), each
// range's float32 sums go to a plane of `partials`, and router_reduce_kernel
// adds the planes in order, then the gate bias. Deterministic; float32
// accumulation throughout.
int router_kparts(const moe_config& c) {
  if (c.act_dtype != MOE_BF16 || c.router_dtype != MOE_BF16 || c.num_experts % 128 != 0 ||
      c.d_model % kGemmAlign != 0 || c.tokens <= 0)
    return 0;
  const int64_t tiles = (c.tokens + 127) / 128 * (c.num_experts / 128);
  const int nk = (int)(c.d_model / 64);
  int kp = 1;
  // about 256 work items (one per CU; 512 were 3 us slower at the DeepSeek-V3
  // shape), each range at least 4 (even) K steps
  while (tiles * kp * 2 <= 256 && nk % (kp * 2) == 0 && nk / (kp * 2) >= 4 &&
         (nk / (kp * 2)) % 2 == 0)
    kp *= 2;
  return kp;
}

__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ P, int kparts,
                                                            int64_t n4, int E,
                                                            const float* __restrict__ bg,
                                                            float* __restrict__ logits) {
  const f32x4* __restrict__ P4 = reinterpret_cast<const f32x4*>(P);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 s = P4[i];
    for (int p = 1; p < kparts; ++p) s += P4[(int64_t)p * n4 + i];
    if (bg) {
      const int e = (int)((i * 4) % E);
      const f32x4 b = {bg[e], bg[e + 1], bg[e + 2], bg[e + 3]};
      s += b;
    }
    reinterpret_cast<f32x4*>(logits)[i] = s;
  }
}

hipError_t launch_router_gemm(const moe_config& c, const void* x, const void* w_gate,
                              const float* b_gate, float* partials, float* logits,
                              hipStream_t s) {
  const int kp = router_kparts(c);
  const int E = c.num_experts, K = (int)c.d_model;
  const int64_t T = c.tokens;
  const int64_t items = (T + 127) / 128 * (E / 128) * kp;
  const int slots = gemm_slots();
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI_PARTIAL, false>),
                     dim3((unsigned)(items < slots ? items : slots)), dim3(256), 0, s,
                     (const bf16*)x, (const bf16*)w_gate, (const bf16*)nullptr, (const float*)nullptr,
                     (const bf16*)nullptr, (const bf16*)nullptr, (const float*)nullptr, 1, 1,
                     (const int32_t*)nullptr, (int)T, (void*)partials, E, K, 0,
                     (const int32_t*)nullptr, kp, (const bf16*)nullptr, 0, 0, 0, (float*)nullptr, 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n4 = T * E / 4;
  const int64_t blocks = (n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048;
  hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, partials, kp,
                     n4, E, b_gate, logits);
  return hipGetLastError();
}

// x's router term of the backward, dlp [T][2E] (dlogits as two bf16 planes)
// times W_g for both halves of K (ksplit = E, W3 = W_g), on the 128 x 128
// kernel with K-major weights over the single group of T rows, float32 out.
hipError_t launch_router_dx_gemm(const moe_config& c, const void* dlp, const void* w_gate, float* xr,
                                 hipStream_t s) {
  const int E = c.num_experts, N = (int)c.d_model;
  const int64_t T = c.tokens;
  const int64_t tiles = (T + 127) / 128 * (N / 128);
  const int slots = gemm_slots();
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI_PARTIAL, false, true>),
                     dim3((unsigned)(tiles < slots ? tiles : slots)), dim3(256), 0, s,
                     (const bf16*)dlp, (const bf16*)w_gate, (const bf16*)w_gate,
                     (const float*)nullptr, (const bf16*)nullptr, (const bf16*)nullptr,
                     (const float*)nullptr, 1, 1, (const int32_t*)nullptr, (int)T, (void*)xr, N,
                     2 * E, 0, (const int32_t*)nullptr, 1, (const bf16*)nullptr, 0, 0, E,
                     (float*)nullptr, 0);
  return hipGetLastError();
}

template <typename ET, bool HB>
static hipError_t up_typed(const moe_config& c, const ET* a, const int32_t* arows,
                           const int32_t* off, const ExpertWeights& w, ET* h, hipStream_t s) {
  const int N = (int)c.d_ff, K = (int)c.d_model;
  switch (c.activation) {
    case MOE_ACT_GELU:
      return gemm_launch<ET, EPI_GELU, HB>(c, a, w.w1, nullptr, w.b1, w.ws1, nullptr, w.bs1, off, h,
                                           N, K, s, arows, nullptr, w.up_packed);
    case MOE_ACT_RELU:
      return gemm_launch<ET, EPI_RELU, HB>(c, a, w.w1, nullptr, w.b1, w.ws1, nullptr, w.bs1, off, h,
                                           N, K, s, arows, nullptr, w.up_packed);
    default:
      return gemm_launch<ET, EPI_SWIGLU, HB>(c, a, w.w1, w.w3, w.b1, w.ws1, w.ws3, w.bs1, off, h, N,
                                             K, s, arows, nullptr, w.up_packed);
  }
}

hipError_t launch_expert_up(const moe_config& c, const void* a, const int32_t* offsets,
                            const ExpertWeights& w, void* h, hipStream_t s, const int32_t* arows) {
  if (c.act_dtype == MOE_BF16)
    return c.has_bias ? up_typed<bf16, true>(c, (const bf16*)a, arows, offsets, w, (bf16*)h, s)
                      : up_typed<bf16, false>(c, (const bf16*)a, arows, offsets, w, (bf16*)h, s);
  return c.has_bias ? up_typed<float, true>(c, (const float*)a, arows, offsets, w, (float*)h, s)
                    : up_typed<float, false>(c, (const float*)a, arows, offsets, w, (float*)h, s);
}

hipError_t launch_expert_down(const moe_config& c, const void* h, const int32_t* offsets,
                              const ExpertWeights& w, void* y_perm, hipStream_t s,
                              void* rest_partial, size_t rest_bytes) {
  const int N = (int)c.d_model, K = (int)c.d_ff;
  float* rp = (float*)rest_partial;
  if (c.act_dtype == MOE_BF16)
    return c.has_bias
               ? gemm_launch<bf16, EPI_NONE, true>(c, (const bf16*)h, w.w2, nullptr, w.b2, w.ws2,
                                                   nullptr, w.bs2, offsets, (bf16*)y_perm, N, K, s,
                                                   nullptr, nullptr, w.down_packed, 0, nullptr, 0,
                                                   rp, rest_bytes)
               : gemm_launch<bf16, EPI_NONE, false>(c, (const bf16*)h, w.w2, nullptr, w.b2, w.ws2,
                                                    nullptr, w.bs2, offsets, (bf16*)y_perm, N, K,
                                                    s, nullptr, nullptr, w.down_packed, 0, nullptr,
                                                    0, rp, rest_bytes);
  return c.has_bias
             ? gemm_launch<float, EPI_NONE, true>(c, (const float*)h, w.w2, nullptr, w.b2, w.ws2,
                                                  nullptr, w.bs2, offsets, (float*)y_perm, N, K, s)
             : gemm_launch<float, EPI_NONE, false>(c, (const float*)h, w.w2, nullptr, w.b2, w.ws2,
                                                   nullptr, w.bs2, offsets, (float*)y_perm, N, K,
                                                   s);
}

// ------------------------------------------------------------------ backward
// W2 [d][F] per group is the K-major B operand of dYp W2 (K = d, N = F).
hipError_t launch_backward_dz(const moe_config& c, const void* dyp, const int32_t* offsets,
                              const void* w2, const void* ws2, const void* z, void* dz,
                              float* colsum, int colsum_tiles, hipStream_t s) {
  const int N = (int)c.d_ff, K = (int)c.d_model;
  if (c.activation == MOE_ACT_GELU)
    return gemm_launch<bf16, EPI_DGELU, false, true>(c, (const bf16*)dyp, w2, nullptr, nullptr, ws2,
                                                     nullptr, nullptr, offsets, (bf16*)dz, N, K, s,
                                                     nullptr, (const bf16*)z, nullptr, K, colsum, colsum_tiles);
  if (c.activation == MOE_ACT_RELU)
    return gemm_launch<bf16, EPI_DRELU, false, true>(c, (const bf16*)dyp, w2, nullptr, nullptr, ws2,
                                                     nullptr, nullptr, offsets, (bf16*)dz, N, K, s,
                                                     nullptr, (const bf16*)z, nullptr, K, colsum, colsum_tiles);
  // SwiGLU: dH itself (the elementwise step forms dz1 and du)
  return gemm_launch<bf16, EPI_NONE, false, true>(c, (const bf16*)dyp, w2, nullptr, nullptr, ws2,
                                                  nullptr, nullptr, offsets, (bf16*)dz, N, K, s,
                                                  nullptr, nullptr, nullptr, K);
}

hipError_t launch_linear_rows(const moe_config& c, const void* a, const int32_t* offsets,
                              const void* W, const float* b, const void* Ws, const float* bs,
                              void* out, int N, int K, hipStream_t s, const int32_t* arows) {
  if (c.act_dtype != MOE_BF16)
    return b ? gemm_launch<float, EPI_NONE, true>(c, (const float*)a, W, nullptr, b, Ws, nullptr,
                                                  bs, offsets, (float*)out, N, K, s, arows)
             : gemm_launch<float, EPI_NONE, false>(c, (const float*)a, W, nullptr, nullptr, Ws,
                                                   nullptr, nullptr, offsets, (float*)out, N, K, s,
                                                   arows);
  return b ? gemm_launch<bf16, EPI_NONE, true>(c, (const bf16*)a, W, nullptr, b, Ws, nullptr, bs,
                                               offsets, (bf16*)out, N, K, s, arows)
           : gemm_launch<bf16, EPI_NONE, false>(c, (const bf16*)a, W, nullptr, nullptr, Ws, nullptr,
                                                nullptr, offsets, (bf16*)out, N, K, s, arows);
}

hipError_t launch_expert_up_linear(const moe_config& c, const void* a, const int32_t* offsets,
                                   const ExpertWeights& w, void* z, hipStream_t s,
                                   const int32_t* arows) {
  const int N = (int)c.d_ff, K = (int)c.d_model;
  hipError_t e = launch_linear_rows(c, a, offsets, w.w1, c.has_bias ? w.b1 : nullptr, w.ws1,
                                    c.has_bias ? w.bs1 : nullptr, z, N, K, s, arows);
  if (e != hipSuccess || c.activation != MOE_ACT_SWIGLU) return e;
  // SwiGLU: the second plane u = x W3^T (no bias)
  const size_t es = c.act_dtype == MOE_BF16 ? 2 : 4;
  return launch_linear_rows(c, a, offsets, w.w3, nullptr, w.ws3, nullptr,
                            (char*)z + (size_t)rows_max(c) * c.d_ff * es, N, K, s, arows);
}

// W1 [F][d] per group is the K-major B operand of dZ W1 (K = F, N = d); for
// SwiGLU the K steps from F on take W3 (dZ = [dz1 | du]).
hipError_t launch_backward_dx(const moe_config& c, const void* dz, const int32_t* offsets,
                              const void* w1, const void* w3, const void* ws1, const void* ws3,
                              void* dxp, hipStream_t s, void* rest_partial, size_t rest_bytes) {
  const int N = (int)c.d_model, F = (int)c.d_ff;
  const bool sw = c.activation == MOE_ACT_SWIGLU;
  return gemm_launch<bf16, EPI_NONE, false, true>(c, (const bf16*)dz, w1, sw ? w3 : nullptr, nullptr,
                                                  ws1, sw ? ws3 : nullptr, nullptr, offsets,
                                                  (bf16*)dxp, N, sw ? 2 * F : F, s, nullptr, nullptr,
                                                  nullptr, F, nullptr, 0, (float*)rest_partial,
                                                  rest_bytes);
}

// The streaming threshold gemm_launch applies: groups of at most kStreamMaxRows
// rows are streamed for the forward epilogues when the A operand spans less
// than 4 GiB; the K-major backward GEMMs stream their groups of at most as
// many rows too (linear epilogue), which only lowers the plan below.
size_t rest_partial_bytes(const moe_config& c, int which) {
  if (c.act_dtype != MOE_BF16) return 0;
  const int N = (int)c.d_model, F = (int)c.d_ff;
  if (which == 0) {
    const int64_t a_span = rows_max(c) * (int64_t)F * 2;
    return rest_split_plan(c, N, F, a_span < ((int64_t)1 << 32) ? kStreamMaxRows : 0).bytes;
  }
  const int K = c.activation == MOE_ACT_SWIGLU ? 2 * F : F;
  return rest_split_plan(c, N, K, 0).bytes;
}

size_t packed_weights_bytes(const moe_config& c, int which) {
  const int64_t G = c.num_experts + c.num_shared_experts;
  const int64_t mats = which == 0 && c.activation == MOE_ACT_SWIGLU ? 2 : 1;
  return (size_t)(G * mats * c.d_ff * c.d_model * 2);
}

hipError_t launch_pack_weights(const moe_config& c, const moe_weights& w, void* up, void* down,
                               hipStream_t s) {
  const int E = c.num_experts, G = c.num_experts + c.num_shared_experts;
  const int F = (int)c.d_ff, d = (int)c.d_model;
  auto grid = [](size_t bytes) {
    const size_t units = bytes / 16;
    const size_t b = (units + 255) / 256;
    return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
  };
  if (up) {
    if (c.activation == MOE_ACT_SWIGLU)
      hipLaunchKernelGGL(pack_weights_kernel<true>, dim3(grid(packed_weights_bytes(c, 0))), dim3(256), 0,
                         s, (const bf16*)w.w1, (const bf16*)w.w3, (const bf16*)w.ws1,
                         (const bf16*)w.ws3, E, G, F, d, (u32x4*)up);
    else
      hipLaunchKernelGGL(pack_weights_kernel<false>, dim3(grid(packed_weights_bytes(c, 0))), dim3(256),
                         0, s, (const bf16*)w.w1, (const bf16*)nullptr, (const bf16*)w.ws1,
                         (const bf16*)nullptr, E, G, F, d, (u32x4*)up);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (down) {
    hipLaunchKernelGGL(pack_weights_kernel<false>, dim3(grid(packed_weights_bytes(c, 1))), dim3(256), 0,
                       s, (const bf16*)w.w2, (const bf16*)nullptr, (const bf16*)w.ws2,
                       (const bf16*)nullptr, E, G, d, F, (u32x4*)down);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_wgrad(const void* a, int lda, const void* b, int ldb, const int32_t* so, int G,
                        int E, int M, int N, int64_t rows, float* C, float* Cs, hipStream_t s) {
  const int64_t tiles = (int64_t)G * (M / 128) * (N / 128);
  if (tiles <= 0) return hipSuccess;
  // 256 x 256 tiles where they number at least one per CU and the groups
  // average at least 512 rows (8 K steps); with fewer rows per group (the
  // DeepSeek-V3 shape: ~140) a tile is mostly its float32 output, which two
  // 128 x 128 blocks per CU overlap with each other's loads
  const int64_t big = M % 256 == 0 && N % 256 == 0 ? (int64_t)G * (M / 256) * (N / 256) : 0;
  if (big >= 256 && rows >= (int64_t)512 * G)
    hipLaunchKernelGGL(gemm_wgrad_tn_big_kernel, dim3((unsigned)big), dim3(256), 0, s,
                       (const bf16*)a, lda, (const bf16*)b, ldb, so, G, E, M, N, C, Cs);
  else
    hipLaunchKernelGGL(gemm_wgrad_tn_kernel, dim3((unsigned)(tiles / wgrad_run(N / 128))), dim3(256),
                       0, s, (const bf16*)a, lda, (const bf16*)b, ldb, so, G, E, M, N, C, Cs);
  return hipGetLastError();
}

}  // namespace moe
