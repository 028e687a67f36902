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

enum { EPI_GELU = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_NONE = 3 };

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
    o[i] = gi <= G ? min(max(offsets[gi], 0), rows_max) : rows_max;
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

// C[r, n] = epi(sum_k A[r, k] W_g[n, k] + b_g[n]) for the rows of each tile.
// Group g < E takes expert weights W + g N K; group E (shared expert) takes Ws.
template <int EPI, bool HAS_BIAS>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* __restrict__ W3,
    const float* __restrict__ bias, const bf16* __restrict__ Ws, const bf16* __restrict__ Ws3,
    const float* __restrict__ bias_s, int E, int G, const int32_t* __restrict__ offsets,
    int rows_max, bf16* __restrict__ C, int N, int K) {
  constexpr bool GATED = EPI == EPI_SWIGLU;
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
  constexpr int CH = BK / 8;           // 16-byte chunks per tile row
  constexpr int NB = GATED ? 2 : 1;    // B operands (W1 and W3 for SwiGLU)
  __shared__ uint4 sA[2][BM * CH];
  __shared__ uint4 sB[NB][2][BN * CH];

  const int ntn = N / BN;
  const int mt = blockIdx.x / ntn;
  const int nt = blockIdx.x - mt * ntn;
  int g, row0, nrows;
  if (!find_tile(offsets, G, rows_max, BM, mt, g, row0, nrows)) return;
  const int n0 = nt * BN;
  const bf16* Wg = g < E ? W + (int64_t)g * N * K : Ws;
  const bf16* W3g = GATED ? (g < E ? W3 + (int64_t)g * N * K : Ws3) : nullptr;
  const float* bg = HAS_BIAS ? (g < E ? bias + (int64_t)g * N : bias_s) : nullptr;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register loads: thread covers chunk (tid & 7) of rows (tid >> 3) + 32 i
  const int lc = tid & 7;
  const int lr = tid >> 3;
  const int64_t a_base = (int64_t)row0 * K + lc * 8;
  const int64_t b_base = (int64_t)(n0 + lr) * K + lc * 8;
  const int64_t a_step[4] = {(int64_t)min(lr, nrows - 1) * K, (int64_t)min(lr + 32, nrows - 1) * K,
                             (int64_t)min(lr + 64, nrows - 1) * K,
                             (int64_t)min(lr + 96, nrows - 1) * K};
  const bf16* Ab = A + a_base;
  const bf16* Bb = Wg + b_base;
  const bf16* B3b = GATED ? W3g + b_base : nullptr;
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3, rc0, rc1, rc2, rc3;
#define MOE_GLOAD(k0)                                                                 \
  do {                                                                                \
    ra0 = *reinterpret_cast<const uint4*>(Ab + a_step[0] + (k0));                     \
    ra1 = *reinterpret_cast<const uint4*>(Ab + a_step[1] + (k0));                     \
    ra2 = *reinterpret_cast<const uint4*>(Ab + a_step[2] + (k0));                     \
    ra3 = *reinterpret_cast<const uint4*>(Ab + a_step[3] + (k0));                     \
    rb0 = *reinterpret_cast<const uint4*>(Bb + (k0));                                 \
    rb1 = *reinterpret_cast<const uint4*>(Bb + (int64_t)32 * K + (k0));               \
    rb2 = *reinterpret_cast<const uint4*>(Bb + (int64_t)64 * K + (k0));               \
    rb3 = *reinterpret_cast<const uint4*>(Bb + (int64_t)96 * K + (k0));               \
    if constexpr (GATED) {                                                            \
      rc0 = *reinterpret_cast<const uint4*>(B3b + (k0));                              \
      rc1 = *reinterpret_cast<const uint4*>(B3b + (int64_t)32 * K + (k0));            \
      rc2 = *reinterpret_cast<const uint4*>(B3b + (int64_t)64 * K + (k0));            \
      rc3 = *reinterpret_cast<const uint4*>(B3b + (int64_t)96 * K + (k0));            \
    }                                                                                 \
  } while (0)
  // rows lr + 32 i share (row & 7) = lr & 7, so one swizzled chunk serves all four
  const int slot = lr * CH + (lc ^ (lr & 7));
#define MOE_LSTORE(buf)                                                               \
  do {                                                                                \
    sA[buf][slot] = ra0;                                                              \
    sA[buf][slot + 32 * CH] = ra1;                                                    \
    sA[buf][slot + 64 * CH] = ra2;                                                    \
    sA[buf][slot + 96 * CH] = ra3;                                                    \
    sB[0][buf][slot] = rb0;                                                           \
    sB[0][buf][slot + 32 * CH] = rb1;                                                 \
    sB[0][buf][slot + 64 * CH] = rb2;                                                 \
    sB[0][buf][slot + 96 * CH] = rb3;                                                 \
    if constexpr (GATED) {                                                            \
      sB[NB - 1][buf][slot] = rc0;                                                    \
      sB[NB - 1][buf][slot + 32 * CH] = rc1;                                          \
      sB[NB - 1][buf][slot + 64 * CH] = rc2;                                          \
      sB[NB - 1][buf][slot + 96 * CH] = rc3;                                          \
    }                                                                                 \
  } while (0)

  f32x16 acc[NB][2][2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.f;

  const int nk = K / BK;
  MOE_GLOAD(0);
  MOE_LSTORE(0);
  __syncthreads();
  const int fr = lane & 31;    // fragment row within a 32-row sub-tile
  const int fk = lane >> 5;    // which 8-wide half of the 16-wide K step
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) MOE_GLOAD((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int ch = s * 2 + fk;
      bf16x8 af[2], bfr[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + fr;
        af[i] = __builtin_bit_cast(bf16x8, sA[cur][r * CH + (ch ^ (r & 7))]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + fr;
#pragma unroll
        for (int b = 0; b < NB; ++b)
          bfr[b][j] = __builtin_bit_cast(bf16x8, sB[b][cur][r * CH + (ch ^ (r & 7))]);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[b][j], acc[b][i][j],
                                                                   0, 0, 0);
    }
    if (more) MOE_LSTORE(cur ^ 1);
    __syncthreads();
  }

#undef MOE_GLOAD
#undef MOE_LSTORE

  // Epilogue. Accumulator register r of a 32x32 tile holds row
  // 8 (r / 4) + 4 (lane / 32) + r % 4 and column lane % 32.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + fr;
    const float bv = HAS_BIAS ? bg[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + i * 32 + (r >> 2) * 8 + fk * 4 + (r & 3);
        if (m < nrows) {
          const float z1 = acc[0][i][j][r] + bv;
          const float z3 = GATED ? acc[NB - 1][i][j][r] : 0.f;
          store1(C + (int64_t)(row0 + m) * N + n, epilogue<EPI>(z1, z3));
        }
      }
    }
  }
}

// float32 layers: one thread per (row, column) of a tile, plain FMA loop.
template <int EPI, bool HAS_BIAS>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ W, const float* __restrict__ W3,
    const float* __restrict__ bias, const float* __restrict__ Ws, const float* __restrict__ Ws3,
    const float* __restrict__ bias_s, int E, int G, const int32_t* __restrict__ offsets,
    int rows_max, float* __restrict__ C, int N, int K) {
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
    const float* a = A + (int64_t)(row0 + m) * K;
    float s1 = 0.f, s3 = 0.f;
    for (int kk = 0; kk < K; ++kk) {
      s1 = fmaf(a[kk], w[kk], s1);
      if (GATED) s3 = fmaf(a[kk], w3[kk], s3);
    }
    C[(int64_t)(row0 + m) * N + n] = epilogue<EPI>(s1 + bv, s3);
  }
}

template <typename ET, int EPI, bool HB>
static hipError_t gemm_launch(const moe_config& c, const ET* A, const void* W, const void* W3,
                              const float* bias, const void* Ws, const void* Ws3,
                              const float* bias_s, const int32_t* offsets, ET* C, int N, int K,
                              hipStream_t s) {
  const int E = c.num_experts, G = c.num_experts + c.num_shared_experts;
  const int64_t rows = rows_max(c);
  const unsigned mtiles = (unsigned)((rows + kGemmBM - 1) / kGemmBM) + G;
  if constexpr (sizeof(ET) == 2) {
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, HB>), dim3(mtiles * (N / kGemmBN)), dim3(256), 0, s,
                       A, (const bf16*)W, (const bf16*)W3, bias, (const bf16*)Ws, (const bf16*)Ws3,
                       bias_s, E, G, offsets, (int)rows, C, N, K);
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<EPI, HB>), dim3(mtiles * ((N + 255) / 256)), dim3(256), 0,
                       s, A, (const float*)W, (const float*)W3, bias, (const float*)Ws,
                       (const float*)Ws3, bias_s, E, G, offsets, (int)rows, C, N, K);
  }
  return hipGetLastError();
}

template <typename ET, bool HB>
static hipError_t up_typed(const moe_config& c, const ET* x_perm, const int32_t* off,
                           const ExpertWeights& w, ET* h, hipStream_t s) {
  const int N = (int)c.d_ff, K = (int)c.d_model;
  switch (c.activation) {
    case MOE_ACT_GELU:
      return gemm_launch<ET, EPI_GELU, HB>(c, x_perm, w.w1, nullptr, w.b1, w.ws1, nullptr, w.bs1,
                                           off, h, N, K, s);
    case MOE_ACT_RELU:
      return gemm_launch<ET, EPI_RELU, HB>(c, x_perm, w.w1, nullptr, w.b1, w.ws1, nullptr, w.bs1,
                                           off, h, N, K, s);
    default:
      return gemm_launch<ET, EPI_SWIGLU, HB>(c, x_perm, w.w1, w.w3, w.b1, w.ws1, w.ws3, w.bs1, off,
                                             h, N, K, s);
  }
}

hipError_t launch_expert_up(const moe_config& c, const void* x_perm, const int32_t* offsets,
                            const ExpertWeights& w, void* h, hipStream_t s) {
  if (c.act_dtype == MOE_BF16)
    return c.has_bias ? up_typed<bf16, true>(c, (const bf16*)x_perm, offsets, w, (bf16*)h, s)
                      : up_typed<bf16, false>(c, (const bf16*)x_perm, offsets, w, (bf16*)h, s);
  return c.has_bias ? up_typed<float, true>(c, (const float*)x_perm, offsets, w, (float*)h, s)
                    : up_typed<float, false>(c, (const float*)x_perm, offsets, w, (float*)h, s);
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

}  // namespace moe
