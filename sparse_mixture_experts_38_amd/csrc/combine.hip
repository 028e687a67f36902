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

template <typename ET>
__global__ __launch_bounds__(256) void combine_kernel(const ET* __restrict__ y_perm,
                                                      const int32_t* __restrict__ expert_offsets,
                                                      const int32_t* __restrict__ assign_row,
                                                      const float* __restrict__ gate, int64_t T,
                                                      int k, int E, int S, int d,
                                                      ET* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int64_t rows[MOE_MAX_TOP_K];
  float g[MOE_MAX_TOP_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K; ++j) {
    rows[j] = -1;
    g[j] = 0.f;
    if (j < k) {
      rows[j] = assign_row[t * k + j];
      g[j] = gate[t * k + j];
    }
  }
  const int64_t srow = S ? (int64_t)expert_offsets[E] + t : -1;
  for (int c = lane * 8; c < d; c += 512) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOP_K; ++j) {
      if (j < k && rows[j] >= 0) {
        float v[8];
        load8(y_perm + rows[j] * d + c, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(g[j], v[q], acc[q]);
      }
    }
    if (srow >= 0) {
      float v[8];
      load8(y_perm + srow * d + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += v[q];
    }
    store8(y + t * d + c, acc);
  }
}

hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* expert_offsets,
                          const int32_t* assign_row, const float* topk_gate, void* y,
                          hipStream_t s) {
  const int64_t T = c.tokens;
  const unsigned blocks = (unsigned)((T + 3) / 4);
  if (c.act_dtype == MOE_BF16)
    hipLaunchKernelGGL((combine_kernel<bf16>), dim3(blocks), dim3(256), 0, s, (const bf16*)y_perm,
                       expert_offsets, assign_row, topk_gate, T, c.top_k, c.num_experts,
                       c.num_shared_experts, (int)c.d_model, (bf16*)y);
  else
    hipLaunchKernelGGL((combine_kernel<float>), dim3(blocks), dim3(256), 0, s,
                       (const float*)y_perm, expert_offsets, assign_row, topk_gate, T, c.top_k,
                       c.num_experts, c.num_shared_experts, (int)c.d_model, (float*)y);
  return hipGetLastError();
}

}  // namespace moe
