// Gate-weighted combine of the expert outputs back into token order.
//
// MoE From Scratch to DeepSeek V3: y = sum over the top-k experts of
// Gate_i(x) E_i(x); shared experts are always active (gate 1). MoE Training:
// Mixture of Experts, "Weighted Combination". Gather form: each token reads
// its k rows (fixed j order, float32 accumulation, one rounding to the output
// type), so there are no atomics and the result is deterministic. Dropped
// assignments (row -1) contribute nothing.
#include "moe_internal.h"

namespace moe {

// KM >= k bounds the per-token row count at compile time. Every row load is
// unconditional so that a lane's loads all issue before the first use (a
// guarded load is followed by its own wait): a slot that is dropped, or past
// k, reads the token's first live row, data that is in flight anyway, and is
// masked out; a token with no live row only stores zeros.
template <typename ET, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const ET* __restrict__ y_perm,
                                                      const int32_t* __restrict__ expert_offsets,
                                                      const int32_t* __restrict__ assign_row,
                                                      const float* __restrict__ gate, int64_t T,
                                                      int k, int E, int S, int d,
                                                      ET* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int64_t rows[KM];
  float g[KM];
  bool live[KM];
  int64_t first = -1;
#pragma unroll
  for (int j = 0; j < KM; ++j) {   // slots past k reread slot k - 1 (unconditional loads)
    const int64_t i = t * k + min(j, k - 1);
    rows[j] = assign_row[i];
    g[j] = gate[i];
    live[j] = j < k && rows[j] >= 0;
  }
#pragma unroll
  for (int j = KM - 1; j >= 0; --j)
    if (live[j]) first = rows[j];
  const int64_t srow = S ? (int64_t)expert_offsets[E] + t : -1;
  if (first < 0) first = srow;
  if (first < 0) {   // every assignment dropped and no shared expert
    float z[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) z[q] = 0.f;
    for (int c = lane * 8; c < d; c += 512) store8(y + t * d + c, z);
    return;
  }
  const ET* src[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) src[j] = y_perm + (live[j] ? rows[j] : first) * d;
  for (int c = lane * 8; c < d; c += 512) {
    float v[KM][8];
#pragma unroll
    for (int j = 0; j < KM; ++j) load8(src[j] + c, v[j]);
    float vs[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) vs[q] = 0.f;
    if (srow >= 0) load8(y_perm + srow * d + c, vs);   // last: its wait covers all loads
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = live[j] ? fmaf(g[j], v[j][q], acc[q]) : acc[q];
    if (srow >= 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += vs[q];
    }
    store8(y + t * d + c, acc);
  }
}

template <typename ET>
static void launch_combine_t(const moe_config& c, const ET* y_perm, const int32_t* expert_offsets,
                             const int32_t* assign_row, const float* topk_gate, ET* y,
                             hipStream_t s) {
  const int64_t T = c.tokens;
  const unsigned blocks = (unsigned)((T + 3) / 4);
  const int k = c.top_k, E = c.num_experts, S = c.num_shared_experts, d = (int)c.d_model;
  if (k <= 1)
    hipLaunchKernelGGL((combine_kernel<ET, 1>), dim3(blocks), dim3(256), 0, s, y_perm,
                       expert_offsets, assign_row, topk_gate, T, k, E, S, d, y);
  else if (k <= 2)
    hipLaunchKernelGGL((combine_kernel<ET, 2>), dim3(blocks), dim3(256), 0, s, y_perm,
                       expert_offsets, assign_row, topk_gate, T, k, E, S, d, y);
  else if (k <= 4)
    hipLaunchKernelGGL((combine_kernel<ET, 4>), dim3(blocks), dim3(256), 0, s, y_perm,
                       expert_offsets, assign_row, topk_gate, T, k, E, S, d, y);
  else
    hipLaunchKernelGGL((combine_kernel<ET, MOE_MAX_TOP_K>), dim3(blocks), dim3(256), 0, s,
                       y_perm, expert_offsets, assign_row, topk_gate, T, k, E, S, d, y);
}

hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* expert_offsets,
                          const int32_t* assign_row, const float* topk_gate, void* y,
                          hipStream_t s) {
  if (c.act_dtype == MOE_BF16)
    launch_combine_t<bf16>(c, (const bf16*)y_perm, expert_offsets, assign_row, topk_gate,
                           (bf16*)y, s);
  else
    launch_combine_t<float>(c, (const float*)y_perm, expert_offsets, assign_row, topk_gate,
                            (float*)y, s);
  return hipGetLastError();
}

}  // namespace moe
