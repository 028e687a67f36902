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
// BM-row tiles.
struct TileSpace {
  int s[5], e[5], n[5];
  int excl, incl, total;
};

__device__ __forceinline__ void tile_space_init(TileSpace& ts, const int32_t* __restrict__ offsets,
                                                int G, int rows_max, int BM, int part = 0,
                                                int big = 256) {
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
    const int rows = (gi < G && o[i + 1] > o[i]) ? o[i + 1] - o[i] : 0;
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
template <int EPI, bool HAS_BIAS>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* __restrict__ W3,
    const float* __restrict__ bias, const bf16* __restrict__ Ws, const bf16* __restrict__ Ws3,
    const float* __restrict__ bias_s, int E, int G, const int32_t* __restrict__ offsets,
    int rows_max, void* __restrict__ Cv, int N, int K, int part, const int32_t* __restrict__ arows,
    int kparts, const bf16* __restrict__ Zin) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
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
  tile_space_init(ts, offsets, G, rows_max, BM, part, kGemmBigBM);
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
  int g, row0, nrows, n0;
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
    tile_lookup(ts, mt, BM, g, row0, nrows);
    // uniform over the block: keep them in scalar registers
    g = __builtin_amdgcn_readfirstlane(g);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    n0 = nt * BN;
    Wg = g < E ? W + (int64_t)g * N * K : Ws;
    W3g = GATED ? (g < E ? W3 + (int64_t)g * N * K : Ws3) : Wg;
    bg = HAS_BIAS ? (g < E ? bias + (int64_t)g * N : bias_s) : nullptr;
    b_s = reinterpret_cast<const char*>(Wg + (int64_t)n0 * K);
    b3_s = GATED ? reinterpret_cast<const char*>(W3g + (int64_t)(n0 - BN) * K) : b_s;
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
  const uint32_t bo0 = (uint32_t)(lr * K + lc * 8) * 2u;
  const uint32_t bo1 = bo0 + (uint32_t)(64 * K);    // + 32 rows
  const uint32_t bo2 = bo0 + (uint32_t)(128 * K);
  const uint32_t bo3 = bo0 + (uint32_t)(192 * K);

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
    if ((i) == 4) R.v4 = *reinterpret_cast<const u32x4*>(b_s + kb_ + bo0);           \
    if ((i) == 5) R.v5 = *reinterpret_cast<const u32x4*>(b_s + kb_ + bo1);           \
    if ((i) == 6) R.v6 = *reinterpret_cast<const u32x4*>(b3_s + kb_ + bo2);          \
    if ((i) == 7) R.v7 = *reinterpret_cast<const u32x4*>(b3_s + kb_ + bo3);          \
  } while (0)
#define MOE_W(R, st, i)                                                              \
  do {                                                                               \
    u32x4* d_ = smem + (st) * STAGE + wslot;                                         \
    if ((i) == 0) d_[0] = R.v0;                                                      \
    if ((i) == 1) d_[32 * CH] = R.v1;                                                \
    if ((i) == 2) d_[64 * CH] = R.v2;                                                \
    if ((i) == 3) d_[96 * CH] = R.v3;                                                \
    if ((i) == 4) d_[BM * CH] = R.v4;                                                \
    if ((i) == 5) d_[(BM + 32) * CH] = R.v5;                                         \
    if ((i) == 6) d_[(BM + 64) * CH] = R.v6;                                         \
    if ((i) == 7) d_[(BM + 96) * CH] = R.v7;                                         \
  } while (0)
#define MOE_R(F, st, s4, f)                                                          \
  F[f] = __builtin_bit_cast(bf16x8, smem[(st) * STAGE + fbase[f] + cidx[s4]])
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
  const int cur_row0 = row0, cur_nrows = nrows, cur_n0 = n0, cur_kp = kp;
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
    // float32 sums straight to plane cur_kp of C ([kparts][rows_max][N]):
    // lane (fr, fk) holds 4 consecutive columns of each 8-column group
    float* __restrict__ Cp = reinterpret_cast<float*>(Cv) + (int64_t)cur_kp * rows_max * N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = wm * 64 + i * 32 + fr;
      if (m < cur_nrows) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x4 v = {acc[i + 2 * j][qd * 4 + 0], acc[i + 2 * j][qd * 4 + 1],
                             acc[i + 2 * j][qd * 4 + 2], acc[i + 2 * j][qd * 4 + 3]};
            *reinterpret_cast<f32x4*>(Cp + (int64_t)(cur_row0 + m) * N + cur_n0 + wn * WN + j * 32 +
                                      qd * 8 + fk * 4) = v;
          }
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
  // backward epilogues: the 4 saved pre-activations of each accumulator quad
  uint2 zv[DACT ? TM : 1][DACT ? TN : 1][4];
  if constexpr (DACT) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = wm * 64 + i * 32 + fr;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          zv[i][j][qd] = m < cur_nrows
                             ? *reinterpret_cast<const uint2*>(Zin + (int64_t)(cur_row0 + m) * N + cur_n0 +
                                                               wn * WN + j * 32 + qd * 8 + fk * 4)
                             : make_uint2(0u, 0u);
    }
  }
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
        float zs[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (DACT) {
          const uint2 u = zv[i][j][qd];
          zs[0] = bf16_bits_to_f32(u.x & 0xffffu); zs[1] = bf16_bits_to_f32(u.x >> 16);
          zs[2] = bf16_bits_to_f32(u.y & 0xffffu); zs[3] = bf16_bits_to_f32(u.y >> 16);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = epilogue_bf16<EPI>(z[e], GATED ? acc[i + 2][qd * 4 + e] : zs[e]);
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

// Weight-gradient GEMM with a ragged K range per group (backward pass): for
// group g,
//   C_g[m, n] = sum over k in [po[g], po[g + 1]) of A[m, k] B[n, k],
// A [M][ldk] and B [N][ldk] bf16 hold the expert-sorted row buffers transposed,
// each group's rows padded with zeros to a multiple of 128 columns (at least
// 128), so every K range is a whole, even number of 64-deep steps. C_g is
// float32 [M][N] at C + g M N for a routed expert (g < E) and Cs for the shared
// expert (g == E). Same 128 x 128 tile, LDS layout, fragment order and two-step
// register pipeline as gemm_bf16_kernel (its macros), one tile per block; the
// XCD-aware order keeps a group's tiles on one XCD in groups of 8 M tiles.
// Requires M, N multiples of 128 and 256 ldk < 2^31 (checked by the host).
__global__ __launch_bounds__(256, 2) void gemm_wgrad_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B, const int32_t* __restrict__ po, int G,
    int E, int M, int N, int ldk, float* __restrict__ C, float* __restrict__ Cs) {
  constexpr int BM = 128, BN = 128, BK = 64, CH = BK / 8;
  constexpr int WN = BN / 2, TM = 2, TN = WN / 32;
  constexpr int ROWS = BM + BN, STAGE = ROWS * CH, GROUP_M = 8;
  __shared__ u32x4 smem[2 * STAGE];
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
  const int row0 = (first_m + in2 % gm) * BM;
  const int n0 = (in2 / gm) * BN;
  const int kbase = po[g] / BK;
  const int len = (po[g + 1] - po[g]) / BK;   // even, >= 2
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31;
  const int fk = lane >> 5;
  const int lr = tid >> 3;
  const int lc = tid & 7;
  const int wslot = lr * CH + (lc ^ ((tid >> 4) & 7));
  const int rsw = (fr >> 1) & 7;
  const bf16* a0 = A + lc * 8;
  const char* ar0 = reinterpret_cast<const char*>(a0 + (int64_t)(row0 + lr) * ldk);
  const char* ar1 = reinterpret_cast<const char*>(a0 + (int64_t)(row0 + lr + 32) * ldk);
  const char* ar2 = reinterpret_cast<const char*>(a0 + (int64_t)(row0 + lr + 64) * ldk);
  const char* ar3 = reinterpret_cast<const char*>(a0 + (int64_t)(row0 + lr + 96) * ldk);
  const char* b_s = reinterpret_cast<const char*>(B + (int64_t)n0 * ldk);
  const char* b3_s = b_s;
  const uint32_t bo0 = (uint32_t)(lr * ldk + lc * 8) * 2u;
  const uint32_t bo1 = bo0 + (uint32_t)(64 * ldk);
  const uint32_t bo2 = bo0 + (uint32_t)(128 * ldk);
  const uint32_t bo3 = bo0 + (uint32_t)(192 * ldk);
  int fbase[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int row = f < 2 ? wm * 64 + f * 32 + fr : BM + wn * WN + (f - 2) * 32 + fr;
    fbase[f] = row * CH;
  }
  constexpr int kRO[4] = {0, 2, 1, 3};
  int cidx[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) cidx[s4] = (s4 * 2 + fk) ^ rsw;
  struct Regs { u32x4 v0, v1, v2, v3, v4, v5, v6, v7; };
  Regs r0, r1;
  bf16x8 fr0[4], fr1[4];
  f32x16 acc[4];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k4][r] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) MOE_G(r0, 0, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) MOE_G(r1, 1, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) MOE_W(r0, 0, i);
  __syncthreads();
  for (int kt = 0; kt < len - 2; kt += 2) {
    MOE_STEP(0, r0, kt + 2, true, r1, true);
    __syncthreads();
    MOE_STEP(1, r1, kt + 3, true, r0, true);
    __syncthreads();
  }
  MOE_STEP(0, r0, 0, false, r1, true);
  __syncthreads();
  MOE_STEP(1, r1, 0, false, r0, false);
  float* __restrict__ Cg = g < E ? C + (int64_t)g * M * N : Cs;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * 64 + i * 32 + fr;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const f32x4 v = {acc[i + 2 * j][qd * 4 + 0], acc[i + 2 * j][qd * 4 + 1],
                         acc[i + 2 * j][qd * 4 + 2], acc[i + 2 * j][qd * 4 + 3]};
        *reinterpret_cast<f32x4*>(Cg + (int64_t)(row0 + m) * N + n0 + wn * WN + j * 32 + qd * 8 +
                                  fk * 4) = v;
      }
  }
#undef MOE_SB
#undef MOE_G
#undef MOE_W
#undef MOE_R
#undef MOE_M
#undef MOE_STEP
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
template <int EPI, bool HAS_BIAS>
__global__ __launch_bounds__(256, 1) void gemm_bf16_big_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* __restrict__ W3,
    const float* __restrict__ bias, const bf16* __restrict__ Ws, const bf16* __restrict__ Ws3,
    const float* __restrict__ bias_s, int E, int G, const int32_t* __restrict__ offsets,
    int rows_max, bf16* __restrict__ C, int N, int K, const int32_t* __restrict__ arows,
    uint32_t a_bytes) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
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
  tile_space_init(ts, offsets, G, rows_max, BM, 1, BM);
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
  const bf16* Wg = g < E ? W + (int64_t)g * N * K : Ws;
  const bf16* W3g = GATED ? (g < E ? W3 + (int64_t)g * N * K : Ws3) : Wg;
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
  }
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
  }
  const int nk = K / BK;   // K is a multiple of 256, so nk >= 4 and even

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
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MOE_LDS(MOE_SM(x) + dl + (i) * 8 * CH), 16, \
                                           doff[i], (uint32_t)(kt) * (BK * 2), 0, 0)
#define MOE_R(F, x, s4, f)                                                           \
  F[f] = __builtin_bit_cast(bf16x8, MOE_SM(x)[fbase[f] + cidx[s4]])
#define MOE_M(F, q)                                                                  \
  acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[4 + ((q) >> 2)], F[(q) & 3], acc[q], 0, 0, 0)
  // wait for this wave's direct-to-LDS loads (vmcnt 0, expcnt and lgkmcnt free)
#define MOE_WAIT_LOADS() __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8))
  // the same but for the two prefetches issued last (vmcnt 2)
#define MOE_WAIT_LOADS_PF() __builtin_amdgcn_s_waitcnt(2 | (7 << 4) | (15 << 8))
#define MOE_PF(kt)                                                                   \
  do {                                                                               \
    const uint32_t o_ = (uint32_t)min((kt), nk - 1) * (BK * 2);                      \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MOE_LDS(pf_lds + wave * 128), 4, pfo[0], o_, 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MOE_LDS(pf_lds + wave * 128 + 64), 4, pfo[1], o_, 0, 0); \
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

// Block slots of the persistent 128 x 128 kernel on the current device: two
// per CU, a multiple of 8 (one share per XCD), cached per device.
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

template <typename ET, int EPI, bool HB>
static hipError_t gemm_launch(const moe_config& c, const ET* A, const void* W, const void* W3,
                              const float* bias, const void* Ws, const void* Ws3,
                              const float* bias_s, const int32_t* offsets, ET* C, int N, int K,
                              hipStream_t s, const int32_t* arows = nullptr,
                              const bf16* zin = nullptr) {
  const int E = c.num_experts, G = c.num_experts + c.num_shared_experts;
  const int64_t rows = rows_max(c);
  if constexpr (sizeof(ET) == 2) {
    constexpr int BNB = EPI == EPI_SWIGLU ? 128 : 256;
    constexpr int BN = EPI == EPI_SWIGLU ? 64 : 128;
    // the 128 x 128 kernel is persistent: at most two blocks per CU, each
    // looping over the tiles (grid bounds below; surplus blocks exit)
    const int slots = gemm_slots();
    // 256 x 256 tiles pay off where the K loop is long or there is no
    // activation: one block per CU leaves the epilogue's VALU work exposed,
    // which two 128 x 128 blocks per CU hide behind each other's MFMAs.
    // gathered A rows (arows) are addressed with 32-bit offsets from the start
    // of x, which the 256 x 256 kernel's buffer loads need below 4 GiB
    const int64_t a_bytes = arows ? c.tokens * (int64_t)K * 2 : 0;
    // (the backward epilogues EPI_DGELU / EPI_DRELU exist in the 128 x 128 kernel only)
    const bool big = rows >= kGemmBigBM && (EPI == EPI_NONE || K >= 2048) &&
                     EPI != EPI_DGELU && EPI != EPI_DRELU && a_bytes < ((int64_t)1 << 32);
    if (big) {
      // full 256-row tiles of each group, then the rows left over (< 256 per
      // group) in 128-row tiles; both grids are bounds, surplus blocks exit
      const unsigned big_tiles = (unsigned)(rows / kGemmBigBM) * (unsigned)(N / BNB);
      if constexpr (EPI != EPI_DGELU && EPI != EPI_DRELU)
        hipLaunchKernelGGL((gemm_bf16_big_kernel<EPI, HB>), dim3(big_tiles), dim3(256), 0, s, A,
                           (const bf16*)W, (const bf16*)W3, bias, (const bf16*)Ws, (const bf16*)Ws3,
                           bias_s, E, G, offsets, (int)rows, C, N, K, arows, (uint32_t)a_bytes);
      // each group leaves at most 255 rows, i.e. at most 2 tiles, and the
      // tiles number at most ceil(rows / 128) + G
      const int64_t rest = (rows + 127) / 128 + G < 2 * G ? (rows + 127) / 128 + G : 2 * G;
      const int64_t rgrid = rest * (N / BN) < slots ? rest * (N / BN) : slots;
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI, HB>), dim3((unsigned)rgrid), dim3(256), 0, s, A,
                         (const bf16*)W, (const bf16*)W3, bias, (const bf16*)Ws, (const bf16*)Ws3,
                         bias_s, E, G, offsets, (int)rows, C, N, K, 2, arows, 1, zin);
    } else {
      const int64_t tiles = ((rows + 127) / 128 + G) * (N / BN);
      const int64_t grid = tiles < slots ? tiles : slots;
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI, HB>), dim3((unsigned)grid), dim3(256), 0, s, A,
                         (const bf16*)W, (const bf16*)W3, bias, (const bf16*)Ws, (const bf16*)Ws3,
                         bias_s, E, G, offsets, (int)rows, C, N, K, 0, arows, 1, zin);
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
  // about 512 work items, each range at least 4 (even) K steps
  while (tiles * kp * 2 <= 512 && nk % (kp * 2) == 0 && nk / (kp * 2) >= 4 &&
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
                     (const int32_t*)nullptr, kp, (const bf16*)nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n4 = T * E / 4;
  const int64_t blocks = (n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048;
  hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, partials, kp,
                     n4, E, b_gate, logits);
  return hipGetLastError();
}

template <typename ET, bool HB>
static hipError_t up_typed(const moe_config& c, const ET* a, const int32_t* arows,
                           const int32_t* off, const ExpertWeights& w, ET* h, hipStream_t s) {
  const int N = (int)c.d_ff, K = (int)c.d_model;
  switch (c.activation) {
    case MOE_ACT_GELU:
      return gemm_launch<ET, EPI_GELU, HB>(c, a, w.w1, nullptr, w.b1, w.ws1, nullptr, w.bs1, off, h,
                                           N, K, s, arows);
    case MOE_ACT_RELU:
      return gemm_launch<ET, EPI_RELU, HB>(c, a, w.w1, nullptr, w.b1, w.ws1, nullptr, w.bs1, off, h,
                                           N, K, s, arows);
    default:
      return gemm_launch<ET, EPI_SWIGLU, HB>(c, a, w.w1, w.w3, w.b1, w.ws1, w.ws3, w.bs1, off, h, N,
                                             K, s, arows);
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
                              const ExpertWeights& w, void* y_perm, hipStream_t s) {
  const int N = (int)c.d_model, K = (int)c.d_ff;
  if (c.act_dtype == MOE_BF16)
    return c.has_bias
               ? gemm_launch<bf16, EPI_NONE, true>(c, (const bf16*)h, w.w2, nullptr, w.b2, w.ws2,
                                                   nullptr, w.bs2, offsets, (bf16*)y_perm, N, K, s)
               : gemm_launch<bf16, EPI_NONE, false>(c, (const bf16*)h, w.w2, nullptr, w.b2, w.ws2,
                                                    nullptr, w.bs2, offsets, (bf16*)y_perm, N, K,
                                                    s);
  return c.has_bias
             ? gemm_launch<float, EPI_NONE, true>(c, (const float*)h, w.w2, nullptr, w.b2, w.ws2,
                                                  nullptr, w.bs2, offsets, (float*)y_perm, N, K, s)
             : gemm_launch<float, EPI_NONE, false>(c, (const float*)h, w.w2, nullptr, w.b2, w.ws2,
                                                   nullptr, w.bs2, offsets, (float*)y_perm, N, K,
                                                   s);
}

// ------------------------------------------------------------------ backward
hipError_t launch_backward_dz(const moe_config& c, const void* dyp, const int32_t* offsets,
                              const void* w2t, const void* ws2t, const void* z, void* dz,
                              hipStream_t s) {
  const int N = (int)c.d_ff, K = (int)c.d_model;
  if (c.activation == MOE_ACT_GELU)
    return gemm_launch<bf16, EPI_DGELU, false>(c, (const bf16*)dyp, w2t, nullptr, nullptr, ws2t,
                                               nullptr, nullptr, offsets, (bf16*)dz, N, K, s,
                                               nullptr, (const bf16*)z);
  if (c.activation == MOE_ACT_RELU)
    return gemm_launch<bf16, EPI_DRELU, false>(c, (const bf16*)dyp, w2t, nullptr, nullptr, ws2t,
                                               nullptr, nullptr, offsets, (bf16*)dz, N, K, s,
                                               nullptr, (const bf16*)z);
  // SwiGLU: dH itself (the elementwise step forms dz1 and du)
  return gemm_launch<bf16, EPI_NONE, false>(c, (const bf16*)dyp, w2t, nullptr, nullptr, ws2t,
                                            nullptr, nullptr, offsets, (bf16*)dz, N, K, s);
}

hipError_t launch_linear_rows(const moe_config& c, const void* a, const int32_t* offsets,
                              const void* W, const float* b, const void* Ws, const float* bs,
                              void* out, int N, int K, hipStream_t s, const int32_t* arows) {
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
  return launch_linear_rows(c, a, offsets, w.w3, nullptr, w.ws3, nullptr,
                            (bf16*)z + rows_max(c) * c.d_ff, N, K, s, arows);
}

hipError_t launch_backward_dx(const moe_config& c, const void* dz, const int32_t* offsets,
                              const void* w1t, const void* ws1t, void* dxp, hipStream_t s) {
  const int N = (int)c.d_model;
  const int K = (int)c.d_ff * (c.activation == MOE_ACT_SWIGLU ? 2 : 1);
  return gemm_launch<bf16, EPI_NONE, false>(c, (const bf16*)dz, w1t, nullptr, nullptr, ws1t, nullptr,
                                            nullptr, offsets, (bf16*)dxp, N, K, s);
}

hipError_t launch_wgrad(const void* a, const void* b, const int32_t* po, int G, int E, int M, int N,
                        int ldk, float* C, float* Cs, hipStream_t s) {
  const int64_t tiles = (int64_t)G * (M / 128) * (N / 128);
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_wgrad_kernel, dim3((unsigned)tiles), dim3(256), 0, s, (const bf16*)a,
                     (const bf16*)b, po, G, E, M, N, ldk, C, Cs);
  return hipGetLastError();
}

}  // namespace moe
