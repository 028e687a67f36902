// Expert-choice routing: every expert takes its C best tokens over the
// transposed [E, T] router scores ("MoE Training: Mixture of Experts",
// "2. Routing Mechanisms", expert choice routing: perfect load balance by
// construction; "MoE From Scratch to DeepSeek V3": tokens may be served by
// several experts or none). Score = the float32 router logit; equal scores go to
// the lower token; an expert's output for a token is weighted by the softmax
// probability p[t, e] over experts; expert e's chosen tokens, in ascending
// token order, fill rows e C .. e C + C - 1, and a shared expert takes rows
// E C .. E C + T - 1. The grouped GEMMs are those of the token-choice path.
#include <string.h>

#include "moe_internal.h"

namespace moe {

// Monotone map of a float32 score onto uint32 (a > b as floats iff key(a) > key(b)).
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Per token: lse[t] = logsumexp of its logits; the (t, e) -> row map cleared to
// -1; with a shared expert, row E C + t takes token t.
__global__ __launch_bounds__(256) void ec_lse_kernel(const float* __restrict__ logits, int64_t T,
                                                     int E, int64_t C, int S,
                                                     float* __restrict__ lse,
                                                     int32_t* __restrict__ token_row,
                                                     int32_t* __restrict__ rows) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float* h = logits + t * E;
  float m = -INFINITY;
  for (int e = 0; e < E; ++e) m = fmaxf(m, h[e]);
  float s = 0.f;
  for (int e = 0; e < E; ++e) s += expf(h[e] - m);
  lse[t] = m + logf(s);
  for (int e = 0; e < E; ++e) token_row[t * E + e] = -1;
  if (S) rows[(int64_t)E * C + t] = (int32_t)t;
}

// Block-wide exclusive prefix of a 0/1 flag over 256 threads (4 wavefronts) via
// ballots; returns the prefix and writes the block total to *total.
__device__ __forceinline__ int block_flag_scan(bool flag, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[wave] = __popcll(bal);
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  *total = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
  __syncthreads();   // wave_tot is reused by the next call
  return before + in_wave;
}

// One block per expert e: the C tokens with the largest key(logits[t][e]), ties
// to the lower token. An exact radix select over four 8-bit digits finds the
// C-th largest key K and how many tokens equal to K to take; one ordered pass
// over the tokens (256 per round, ballot scans) then writes the chosen tokens in
// ascending order: tokens[e][i] = t, gates[e][i] = p[t][e], token_row[t][e] =
// e C + i, rows[e C + i] = t. It also writes P_e (mean of p[t][e], float64
// tree) and the balance counts of expert e into stats.
__global__ __launch_bounds__(256) void ec_select_kernel(
    const float* __restrict__ logits, const float* __restrict__ lse, int64_t T, int E, int64_t C,
    int32_t* __restrict__ tokens, float* __restrict__ gates, int32_t* __restrict__ token_row,
    int32_t* __restrict__ rows, moe_stats* __restrict__ stats) {
  __shared__ int hist[256];
  __shared__ int wave_tot[4];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  __shared__ double red[256];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int remaining = (int)C;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int64_t t = tid; t < T; t += 256) {
      const uint32_t u = score_key(logits[t * E + e]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, D = 0;
      for (int dg = 255; dg >= 0; --dg) {
        if (cum + hist[dg] >= remaining) {
          D = dg;
          break;
        }
        cum += hist[dg];
      }
      s_prefix = prefix | ((uint32_t)D << shift);
      s_remaining = remaining - cum;
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 0xFFu << shift;
  }
  // prefix = K; remaining = tokens with key == K to take (lowest tokens first)
  int taken_base = 0, eq_base = 0;
  double psum = 0.0;
  for (int64_t t0 = 0; t0 < T; t0 += 256) {
    const int64_t t = t0 + tid;
    uint32_t u = 0;
    float p = 0.f;
    if (t < T) {
      const float h = logits[t * E + e];
      u = score_key(h);
      p = expf(h - lse[t]);
      psum += (double)p;
    }
    const bool gt = t < T && u > prefix;
    const bool eq = t < T && u == prefix;
    int eq_total = 0;
    const int eq_rank = eq_base + block_flag_scan(eq, wave_tot, &eq_total);
    const bool take = gt || (eq && eq_rank < remaining);
    int take_total = 0;
    const int pos = taken_base + block_flag_scan(take, wave_tot, &take_total);
    if (take && pos < C) {
      const int64_t r = (int64_t)e * C + pos;
      tokens[r] = (int32_t)t;
      gates[r] = p;
      token_row[t * E + e] = (int32_t)r;
      rows[r] = (int32_t)t;
    }
    eq_base += eq_total;
    taken_base += take_total;
  }
  red[tid] = psum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    stats->prob_mean[e] = (float)(red[0] / (double)T);
    stats->counts_pre[e] = (int32_t)C;
    stats->counts_kept[e] = (int32_t)C;
    stats->frac[e] = (float)(1.0 / (double)E);
  }
}

// One block: group offsets (e C; the shared group after E C), the z-loss, the
// number of tokens no expert chose (reported as "dropped"), L_aux from the P_i
// (= sum_i P_i, since every f_i = 1 / E), zeroed unused expert slots.
__global__ __launch_bounds__(256) void ec_finalize_kernel(const float* __restrict__ lse,
                                                          const int32_t* __restrict__ token_row,
                                                          int64_t T, int E, int64_t C, int S,
                                                          int32_t* __restrict__ offsets,
                                                          moe_stats* __restrict__ stats) {
  __shared__ double red[256];
  __shared__ int cnt[256];
  const int tid = threadIdx.x;
  for (int g = tid; g <= E + S; g += 256)
    offsets[g] = (int32_t)(g <= E ? (int64_t)g * C : (int64_t)E * C + T);
  for (int e = E + tid; e < MOE_MAX_EXPERTS; e += 256) {
    stats->counts_pre[e] = 0;
    stats->counts_kept[e] = 0;
    stats->frac[e] = 0.f;
    stats->prob_mean[e] = 0.f;
  }
  double z = 0.0;
  int unpicked = 0;
  for (int64_t t = tid; t < T; t += 256) {
    const double l = (double)lse[t];
    z += l * l;
    bool any = false;
    for (int e = 0; e < E; ++e) any |= token_row[t * E + e] >= 0;
    unpicked += any ? 0 : 1;
  }
  red[tid] = z;
  cnt[tid] = unpicked;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      red[tid] += red[tid + w];
      cnt[tid] += cnt[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    double laux = 0.0;
    for (int e = 0; e < E; ++e) laux += (double)stats->prob_mean[e];
    stats->z_loss = (float)(red[0] / (double)T);
    stats->l_aux = (float)laux;   // E sum_i f_i P_i with f_i = 1 / E
    stats->capacity = (int32_t)C;
    stats->kept = (int32_t)((int64_t)E * C);
    stats->dropped = cnt[0];
  }
}

// y[t] = sum over experts e (ascending) with token_row[t][e] = r >= 0 of
// gates[r] y_perm[r], plus y_perm[E C + t] with a shared expert; float32 sums,
// one rounding. One wavefront per token, 8 columns per lane and step.
template <typename T_>
__global__ __launch_bounds__(256) void ec_combine_kernel(const T_* __restrict__ y_perm,
                                                         const int32_t* __restrict__ token_row,
                                                         const float* __restrict__ gates,
                                                         int64_t T, int d, int E, int64_t C, int S,
                                                         T_* __restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int64_t nrows = (int64_t)E * C;
  for (int c = lane * 8; c < d; c += 512) {
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int e = 0; e < E; ++e) {
      const int r = token_row[t * E + e];
      if (r < 0 || r >= nrows) continue;
      const float g = gates[r];
      float a[8];
      load8(y_perm + (int64_t)r * d + c, a);
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = fmaf(g, a[u], v[u]);
    }
    if (S) {
      float a[8];
      load8(y_perm + (nrows + t) * d + c, a);
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] += a[u];
    }
    store8(y + t * d + c, v);
  }
}

int64_t expert_choice_capacity(const moe_config& c, int64_t token_choice_capacity) {
  int64_t C = token_choice_capacity;
  if (C < 0) C = (c.top_k * c.tokens + c.num_experts - 1) / c.num_experts;
  return C < c.tokens ? C : c.tokens;
}

EcLayout expert_choice_layout(const moe_config& c, int64_t C) {
  EcLayout L;
  memset(&L, 0, sizeof(L));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const int64_t T = c.tokens;
  const int E = c.num_experts, S = c.num_shared_experts;
  // the grouped GEMMs see a layer whose k covers the E C expert rows
  L.gemm_cfg = c;
  L.gemm_cfg.top_k = (int32_t)(T > 0 ? (E * C + T - 1) / T : 1);
  if (L.gemm_cfg.top_k < 1) L.gemm_cfg.top_k = 1;
  L.rows = rows_max(L.gemm_cfg);
  L.logits = take((size_t)T * E * 4);
  L.router_planes = take((size_t)router_kparts(c) * T * E * 4);
  L.lse = take((size_t)T * 4);
  L.row_token = take((size_t)L.rows * 4);
  L.offsets = take((size_t)(E + S + 1) * 4);
  const size_t es = c.act_dtype == MOE_BF16 ? 2 : 4;
  L.h = take((size_t)L.rows * c.d_ff * es);
  L.y_perm = take((size_t)L.rows * c.d_model * es);
  L.total = off;
  return L;
}

hipError_t launch_expert_choice_forward(const moe_config& c, const EcLayout& L, int64_t C,
                                        const void* x, const moe_weights& w, void* y,
                                        const moe_ec_routing& r, moe_stats* stats, char* ws,
                                        hipStream_t s) {
  const int64_t T = c.tokens;
  const int E = c.num_experts, S = c.num_shared_experts;
  float* lg = r.logits ? r.logits : (float*)(ws + L.logits);
  float* lse = (float*)(ws + L.lse);
  int32_t* rows = (int32_t*)(ws + L.row_token);
  int32_t* off = (int32_t*)(ws + L.offsets);
  hipError_t e = launch_router_logits(c, x, w.w_gate, w.b_gate, lg, (float*)(ws + L.router_planes), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ec_lse_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s,
                     (const float*)lg, T, E, C, S, lse, r.token_row, rows);
  hipLaunchKernelGGL(ec_select_kernel, dim3(E), dim3(256), 0, s, (const float*)lg,
                     (const float*)lse, T, E, C, r.tokens, r.gates, r.token_row, rows, stats);
  hipLaunchKernelGGL(ec_finalize_kernel, dim3(1), dim3(256), 0, s, (const float*)lse,
                     (const int32_t*)r.token_row, T, E, C, S, off, stats);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const ExpertWeights ew{w.w1, w.w3, w.w2, w.b1, w.b2, w.ws1, w.ws3, w.ws2, w.bs1, w.bs2};
  void* h = ws + L.h;
  void* yp = ws + L.y_perm;
  e = launch_expert_up(L.gemm_cfg, x, off, ew, h, s, rows);
  if (e != hipSuccess) return e;
  e = launch_expert_down(L.gemm_cfg, h, off, ew, yp, s);
  if (e != hipSuccess) return e;
  const unsigned tb = (unsigned)((T + 3) / 4);
  const int d = (int)c.d_model;
  if (c.act_dtype == MOE_BF16)
    hipLaunchKernelGGL((ec_combine_kernel<bf16>), dim3(tb), dim3(256), 0, s, (const bf16*)yp,
                       (const int32_t*)r.token_row, (const float*)r.gates, T, d, E, C, S, (bf16*)y);
  else
    hipLaunchKernelGGL((ec_combine_kernel<float>), dim3(tb), dim3(256), 0, s, (const float*)yp,
                       (const int32_t*)r.token_row, (const float*)r.gates, T, d, E, C, S,
                       (float*)y);
  return hipGetLastError();
}

}  // namespace moe
