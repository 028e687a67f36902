// Two routing additions around the token-choice path: the selection-bias update
// of auxiliary-loss-free balancing ("MoE From Scratch to DeepSeek V3": b_i is
// lowered for an overloaded expert and raised for an idle one) and hash routing
// (the "Moe(Mixtrue of Experts)" survey: a token -> expert map fixed in advance
// replaces the gating network).
#include "moe_internal.h"

namespace moe {

// b_i <- b_i - gamma sign(c_i E - T k): c_i = top-k picks of expert i before
// capacity (stats->counts_pre), compared with the mean load T k / E exactly in
// integers; float32 arithmetic.
__global__ void bias_update_kernel(const moe_stats* __restrict__ stats, int E, int64_t Tk,
                                   float gamma, float* __restrict__ e_bias) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t v = (int64_t)stats->counts_pre[e] * E - Tk;
  const float s = v > 0 ? 1.f : (v < 0 ? -1.f : 0.f);
  e_bias[e] = e_bias[e] - gamma * s;
}

// topk_idx[t] = table[id] (k = 1), topk_gate[t] = 1; ids outside [0, V) and
// table entries outside [0, E) are clamped. Block 0 also writes P_i = 0 and
// z = 0 (there is no router), which moe_permute's L_aux then reads.
__global__ __launch_bounds__(256) void hash_route_kernel(const int32_t* __restrict__ ids,
                                                         const int32_t* __restrict__ table,
                                                         int64_t V, int64_t T, int E,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_gate,
                                                         moe_stats* __restrict__ stats) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < MOE_MAX_EXPERTS; e += blockDim.x) stats->prob_mean[e] = 0.f;
    if (threadIdx.x == 0) stats->z_loss = 0.f;
  }
  if (t >= T) return;
  int64_t id = ids[t];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  int e = table[id];
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  topk_idx[t] = e;
  topk_gate[t] = 1.f;
}

hipError_t launch_bias_update(const moe_config& c, const moe_stats* stats, float* e_bias,
                              float gamma, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((c.num_experts + 255) / 256), dim3(256), 0, s, stats,
                     c.num_experts, c.tokens * (int64_t)c.top_k, gamma, e_bias);
  return hipGetLastError();
}

hipError_t launch_hash_route(const moe_config& c, const int32_t* ids, const int32_t* table,
                             int64_t V, int32_t* topk_idx, float* topk_gate, moe_stats* stats,
                             hipStream_t s) {
  const int64_t blocks = (c.tokens + 255) / 256;
  hipLaunchKernelGGL(hash_route_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s,
                     ids, table, V, (int64_t)c.tokens, c.num_experts, topk_idx, topk_gate, stats);
  return hipGetLastError();
}

}  // namespace moe
