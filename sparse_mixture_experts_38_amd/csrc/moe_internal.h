// Internal declarations shared by the HIP sources of the MoE library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16-byte register value

constexpr int kWave = 64;

// Assignments ranked per block by the dispatch histogram kernel.
constexpr int kRankChunk = 1024;

// Row tile of the float32 expert GEMM; the bf16 GEMM needs d_model and d_ff to
// be multiples of kGemmAlign (its 256-wide N tiles and 64-deep K steps). The
// bf16 GEMM covers each expert's first floor(rows / kGemmBigBM) * kGemmBigBM
// rows with 256 x 256 tiles and the rest with 128 x 128 tiles.
constexpr int kGemmBM = 128;
constexpr int kGemmBigBM = 256;
constexpr int kGemmAlign = 256;

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bfloat16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  bf16 b = (bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Two float32 -> bfloat16 (round to nearest even), lo in bits 0..15 and hi in
// bits 16..31: one v_cvt_pk_bf16_f32 on gfx950.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_bits_to_f32(u.x & 0xffffu); v[1] = bf16_bits_to_f32(u.x >> 16);
  v[2] = bf16_bits_to_f32(u.y & 0xffffu); v[3] = bf16_bits_to_f32(u.y >> 16);
  v[4] = bf16_bits_to_f32(u.z & 0xffffu); v[5] = bf16_bits_to_f32(u.z >> 16);
  v[6] = bf16_bits_to_f32(u.w & 0xffffu); v[7] = bf16_bits_to_f32(u.w >> 16);
}

__device__ __forceinline__ void store8(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ void store8(bf16* p, const float v[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

__device__ __forceinline__ void store1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store1(bf16* p, float v) {
  *reinterpret_cast<uint16_t*>(p) = f32_to_bf16_bits(v);
}

// Expert activations. GELU is the exact erf form of nn.GELU().
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Phi(-a), the standard normal tail, for a in [0, 6] as 2^P(a): P is a degree-7
// polynomial fitted to log2 Phi(-a) on [0, 6] by least squares (csrc/gelu_fit.py
// prints the fit and its error). Seven FMAs and one hardware exp2.
__device__ __forceinline__ float phi_neg_poly(float a) {
  float p = fmaf(-1.9449223600531695e-06f, a, 6.386057066265494e-05f);
  p = fmaf(p, a, -0.0009488713694736362f);
  p = fmaf(p, a, 0.008582375012338161f);
  p = fmaf(p, a, -0.0541183240711689f);
  p = fmaf(p, a, -0.4582974314689636f);
  p = fmaf(p, a, -1.1513246297836304f);
  p = fmaf(p, a, -0.9999869465827942f);
  return __builtin_amdgcn_exp2f(p);
}

// GELU(x) = x Phi(x) = max(x, 0) - a Phi(-a) with a = |x| clamped to 6 (where
// a Phi(-a) < 1e-8): max absolute error 1e-6 and relative error 1e-5 of the
// GELU. Used where the result is rounded to bf16 (relative step 2^-8).
__device__ __forceinline__ float gelu_poly(float x) {
  const float a = fminf(fabsf(x), 6.0f);
  return fmaf(-a, phi_neg_poly(a), fmaxf(x, 0.f));
}

// d/dx GELU(x) = Phi(x) + x phi(x), with Phi from the same fit (Phi(x) =
// 1 - Phi(-x) for x >= 0) and phi(x) = 2^(-x^2 log2(e) / 2) / sqrt(2 pi).
// Absolute error below 1e-5.
__device__ __forceinline__ float gelu_grad_poly(float x) {
  const float a = fminf(fabsf(x), 6.0f);
  const float q = phi_neg_poly(a);
  const float Phi = x >= 0.f ? 1.0f - q : q;
  const float dens = 0.3989422804014327f * __builtin_amdgcn_exp2f(-0.7213475204444817f * x * x);
  return fmaf(x, dens, Phi);
}

// ------------------------------------------------------------------ workspace
struct WsLayout {
  size_t logits;          // float [T][E] (when the caller does not keep them)
  size_t route_partials;  // float [route_blocks][E + 1]
  size_t router_planes;   // float [router_kparts][T][E] (MFMA router only)
  size_t chunk_hist;      // int32 [chunks][E]
  size_t chunk_base;      // int32 [chunks][E]
  size_t local_rank;      // int32 [T k]
  size_t h;               // act [rows_max][F]
  size_t rest_partial;    // float planes of GEMM 2's split left-over rows (rest_bytes)
  size_t y_perm;          // act [rows_max][d]
  size_t end_route, end_permute, end_ffn, total, rest_bytes;
  int route_blocks, route_iters, chunks;
  int64_t rows_max;
};

WsLayout workspace_layout(const moe_config& c);

// Split along K of the tiled path's left-over rows (groups of more than
// 1536 rows leave up to 255 rows past their full 256-row tiles): kparts float32
// planes of up to cap 128-row tiles, bytes in all (kparts 1: no split).
struct RestSplit {
  int kparts, cap;
  size_t bytes;
};
RestSplit rest_split_plan(const moe_config& c, int N, int K, int skip);
// Bytes of those planes for GEMM 2 of the forward (which 0) or the backward's
// dX GEMM (which 1); 0 where that GEMM does not split.
size_t rest_partial_bytes(const moe_config& c, int which);

// Lanes of a wavefront that cooperate on one token in the top-k kernel.
int route_lanes(int E);

inline int64_t rows_max(const moe_config& c) {
  return c.tokens * c.top_k + (int64_t)c.num_shared_experts * c.tokens;
}

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the first launch error. All enqueue on `stream`.
// Router logits on MFMA (bf16 x and W_g, E a multiple of 128): router_kparts
// is the number of K ranges (0 where this path does not apply), partials holds
// router_kparts planes of T x E float32.
int router_kparts(const moe_config& c);
hipError_t launch_router_gemm(const moe_config& c, const void* x, const void* w_gate,
                              const float* b_gate, float* partials, float* logits,
                              hipStream_t stream);

// Router logits alone (VALU kernel, or the MFMA path with its partial planes).
hipError_t launch_router_logits(const moe_config& c, const void* x, const void* w_gate,
                                const float* b_gate, float* logits, float* router_planes,
                                hipStream_t stream);

// With defer_stats non-null the reduction of the router's per-block partials
// into P_i and z is left to launch_permute (the number of partial rows is
// written to *defer_stats), which then runs it inside its first launch.
hipError_t launch_route(const moe_config& c, const WsLayout& L, const void* x, const void* w_gate,
                        const float* b_gate, const float* e_bias, float* logits, int32_t* topk_idx,
                        float* topk_gate, moe_stats* stats, char* ws, hipStream_t stream,
                        int* defer_stats = nullptr);

// route_blocks > 0: also reduce that many rows of the router's partials (a
// launch_route with defer_stats) into P_i and z, before the statistics that
// need them.
hipError_t launch_permute(const moe_config& c, const WsLayout& L, int64_t capacity,
                          const int32_t* topk_idx, const void* x, int32_t* expert_offsets,
                          int32_t* row_token, int32_t* assign_row, void* x_perm, moe_stats* stats,
                          char* ws, hipStream_t stream, int route_blocks = 0);

// Column col of the router statistics (one block of 256 threads): P_col =
// (1/T) sum of the nblocks per-block partials of column col (col < E), z =
// (1/T) sum of the lse^2 column (col == E), or the zero fill of the unused
// expert slots (col == E + 1); a strided float64 pass per thread, then a tree
// in LDS: deterministic. red: 256 doubles of LDS.
__device__ __forceinline__ void route_stats_column(const float* __restrict__ partials, int nblocks,
                                                   int E, int64_t T, moe_stats* __restrict__ stats,
                                                   int col, double* red) {
  const int tid = threadIdx.x;
  if (col == E + 1) {
    for (int e = E + tid; e < MOE_MAX_EXPERTS; e += 256) stats->prob_mean[e] = 0.f;
    return;
  }
  double s = 0.0;
  for (int b = tid; b < nblocks; b += 256) s += partials[(int64_t)b * (E + 1) + col];
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    const float v = (float)(red[0] / (double)T);
    if (col < E) stats->prob_mean[col] = v;
    else stats->z_loss = v;
  }
}

struct ExpertWeights {
  const void *w1, *w3, *w2;
  const float *b1, *b2;
  const void *ws1, *ws3, *ws2;
  const float *bs1, *bs2;
  // packed copies (moe_pack_weights) read by the weight-streaming GEMM, or null
  const void* up_packed = nullptr;
  const void* down_packed = nullptr;
};

// Bytes of the packed weight copy of GEMM 1 (which = 0: W1, W3) or GEMM 2
// (which = 1: W2) over every group, and the kernels that write them.
size_t packed_weights_bytes(const moe_config& c, int which);
hipError_t launch_pack_weights(const moe_config& c, const moe_weights& w, void* up, void* down,
                               hipStream_t stream);

// Grouped GEMM 1 with the fused activation: h = act(a W1^T + b1) per group, where
// row r of the group's input is row r of a or, with arows, row arows[r] of a.
hipError_t launch_expert_up(const moe_config& c, const void* a, const int32_t* expert_offsets,
                            const ExpertWeights& w, void* h, hipStream_t stream,
                            const int32_t* arows = nullptr);

// Grouped GEMM 2: y_perm = h W2^T + b2 per group (rest_partial: rest_bytes of
// workspace for the split left-over rows, or null).
hipError_t launch_expert_down(const moe_config& c, const void* h, const int32_t* expert_offsets,
                              const ExpertWeights& w, void* y_perm, hipStream_t stream,
                              void* rest_partial = nullptr, size_t rest_bytes = 0);

hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* expert_offsets,
                          const int32_t* assign_row, const float* topk_gate, void* y,
                          hipStream_t stream);

// ------------------------------------------------------------------ balancing, hash routing
hipError_t launch_bias_update(const moe_config& c, const moe_stats* stats, float* e_bias,
                              float gamma, hipStream_t stream);
hipError_t launch_hash_route(const moe_config& c, const int32_t* ids, const int32_t* table,
                             int64_t table_size, int32_t* topk_idx, float* topk_gate,
                             moe_stats* stats, hipStream_t stream);

// ------------------------------------------------------------------ expert choice
// Workspace of moe_forward_expert_choice (byte offsets); gemm_cfg is the layer
// with top_k raised so that its row space T k + S T covers the E C expert rows.
struct EcLayout {
  moe_config gemm_cfg;
  int64_t rows;
  size_t logits, router_planes, lse, zpart, row_token, offsets, h, y_perm, total;
};
// C = the token-choice capacity (or ceil(k T / E) without a limit), at most T.
int64_t expert_choice_capacity(const moe_config& c, int64_t token_choice_capacity);
EcLayout expert_choice_layout(const moe_config& c, int64_t C);
hipError_t launch_expert_choice_forward(const moe_config& c, const EcLayout& L, int64_t C,
                                        const void* x, const moe_weights& w, void* y,
                                        const moe_ec_routing& r, moe_stats* stats, char* ws,
                                        hipStream_t stream);

// ------------------------------------------------------------------ backward
// Workspace of moe_backward (byte offsets). ldk is the length of the padded
// row space of the bias column sums (each group's rows rounded up to a multiple
// of 128, at least 128); xp holds the expert-sorted x rows.
// gate_mfma: the router's backward terms on MFMA (router_bwd_mfma): dlp the
// two bf16 planes of dlogits [T][2E], xr x's router term [T][d] float32, gso
// the gate_slices + 1 token-slice bounds of the router weight gradient.
struct BwdLayout {
  size_t dyp, dgate, dlogits, dz, dh, dxp, po;   // po: padded then sanitized offsets
  size_t xp, colsum1, colsum2, gate_partial, rest_partial, rest_bytes, total;
  size_t dlp, xr, gso;
  int64_t ldk;
  int gate_slices, gate_slice_len, gate_mfma;
};
BwdLayout backward_layout(const moe_config& c);

// Training forward: z = a W1^T + b1 per group (no activation; SwiGLU: a second
// plane u = a W3^T after rows_max x F elements), then h = act(z) (silu(z) u).
hipError_t launch_expert_up_linear(const moe_config& c, const void* a, const int32_t* expert_offsets,
                                   const ExpertWeights& w, void* z, hipStream_t stream,
                                   const int32_t* arows);
hipError_t launch_act_rows(const moe_config& c, const void* z, const int32_t* expert_offsets,
                           void* h, hipStream_t stream);
// Backward steps shared by the bf16 and float32 paths: combine (dYp, dgate),
// router (dlogits), and the gate-bias gradient with dx.
hipError_t launch_combine_backward(const moe_config& c, const void* dy, const void* y_perm,
                                   const moe_routing& r, void* dyp, float* dgate, hipStream_t s);
hipError_t launch_router_backward(const moe_config& c, const moe_routing& r, const moe_stats* stats,
                                  const float* dgate, float aux_coef, float z_coef, float* dlogits,
                                  hipStream_t s);
// (xr: x's router term precomputed, [T][d] float32, or null: computed here)
hipError_t launch_router_bias_and_dx(const moe_config& c, const float* dlogits, const void* dxp,
                                     const moe_routing& r, const moe_weights& w,
                                     const moe_grads& gr, hipStream_t s,
                                     const float* xr = nullptr);
// float32 layers: h = act(z) of the training forward, the backward workspace
// layout (dyp, dgate, dlogits, dz, dh, dxp) and the whole backward.
hipError_t launch_act_rows_f32(const moe_config& c, const void* z, const int32_t* expert_offsets,
                               void* h, hipStream_t stream);
BwdLayout backward_layout_f32(const moe_config& c);
hipError_t launch_backward_f32(const moe_config& c, const BwdLayout& B, const void* x,
                               const moe_weights& w, const moe_routing& r, const moe_stats* stats,
                               const moe_saved& sv, const void* dy, float aux_coef, float z_coef,
                               const moe_grads& gr, char* ws, hipStream_t stream);
// The non-GEMM steps of the backward: phase 0 (combine and router backward,
// padded offsets) before the dZ / dX GEMMs, phase 1 (the expert-sorted x rows,
// weight, bias and router gradients, dx) after them.
hipError_t launch_backward_misc(const moe_config& c, const BwdLayout& B, const void* x,
                                const moe_weights& w, const moe_routing& r, const moe_stats* stats,
                                const moe_saved& sv, const void* dy, float aux_coef, float z_coef,
                                const moe_grads& gr, char* ws, hipStream_t stream, int phase);

// dZ = (dYp W2) * act'(z) per group: dYp [rows][d], W2 [E][d][F] and Ws2 [d][F]
// (the shared expert) as stored, z and dZ [rows][F] bf16 (GELU, ReLU); for
// SwiGLU the product dH = dYp W2 alone, which launch_dswiglu turns into
// dZ = [dz1 | du]. GELU / ReLU with colsum != nullptr: also the column sums of
// each 128-row M tile of dZ, colsum[mt][F] (mt: the tile's index in group
// order, ceil(rows_g / 128) tiles per group; colsum_tiles_reduce_kernel adds
// them per group) for the tiles mt < colsum_tiles.
hipError_t launch_backward_dz(const moe_config& c, const void* dyp, const int32_t* expert_offsets,
                              const void* w2, const void* ws2, const void* z, void* dz,
                              float* colsum, int colsum_tiles, hipStream_t stream);
// dXp = dZ W1 per group (SwiGLU: [dz1 | du] [W1; W3], K = 2F): W1, W3 [E][F][d]
// and Ws1, Ws3 [F][d] as stored; dXp [rows][d] bf16.
hipError_t launch_dswiglu(const moe_config& c, const void* dh, const void* z, void* dz,
                          const int32_t* expert_offsets, hipStream_t stream);
hipError_t launch_backward_dx(const moe_config& c, const void* dz, const int32_t* expert_offsets,
                              const void* w1, const void* w3, const void* ws1, const void* ws3,
                              void* dxp, hipStream_t stream, void* rest_partial = nullptr,
                              size_t rest_bytes = 0);
// Grouped weight gradient over the rows of each group,
// C_g = A[so[g]:so[g+1], 0:M]^T B[so[g]:so[g+1], 0:N]: A [rows][lda], B [rows][ldb]
// bf16 row-major (rows: the rows of all groups, for the choice of tile);
// C float32 [E][M][N], Cs [M][N] for group E.
hipError_t launch_wgrad(const void* a, int lda, const void* b, int ldb, const int32_t* so, int G,
                        int E, int M, int N, int64_t rows, float* C, float* Cs, hipStream_t stream);
// n tiles of 128 columns that one block of the 128 x 128 weight-gradient
// kernel runs in turn (ntn = N / 128 tiles in a row of its output).
__host__ __device__ inline int wgrad_run(int ntn) {
  return ntn % 4 == 0 ? 4 : (ntn % 2 == 0 ? 2 : 1);
}
// The router's backward terms on MFMA where its weights are bf16 and E is a
// multiple of 128 (the layers whose router GEMM runs on MFMA in the forward).
inline bool router_bwd_mfma(const moe_config& c) {
  return c.act_dtype == MOE_BF16 && c.router_dtype == MOE_BF16 && c.num_experts % 128 == 0 &&
         c.tokens > 0;
}
// x's router term xr [T][d] float32 = dlp [T][2E] times W_g (both K halves;
// W_g [E][d] bf16 as stored, K-major).
hipError_t launch_router_dx_gemm(const moe_config& c, const void* dlp, const void* w_gate, float* xr,
                                 hipStream_t stream);

}  // namespace moe
