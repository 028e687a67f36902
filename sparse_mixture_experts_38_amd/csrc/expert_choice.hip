// Expert-choice routing: every expert takes its C best tokens over the
// transposed [E, T] router scores ("MoE Training: Mixture of Experts",
// "2. Routing Mechanisms", expert choice routing: perfect load balance by
// construction; "MoE From Scratch to DeepSeek V3": tokens may be served by
// several experts or none). Key = the float32 router logit (softmax and sigmoid
// scores both increase with it); equal keys go to the lower token; an expert's
// output for a token is weighted by the router score g[t, e]: the softmax
// probability p[t, e] over experts, or the sigmoid score itself (DeepSeek-V3
// scores, no renormalisation over a token's picks); expert e's chosen tokens, in ascending
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

// Per token: norm[t] = logsumexp of its logits (softmax), or the float32 sum
// over experts, in ascending order, of its sigmoid scores (sigmoid); the
// (t, e) -> row map cleared to -1; with a shared expert, row E C + t takes
// token t. Each block writes the float64 sum of its tokens' lse^2 to
// zpart[block] (z-loss, for both score functions).
__global__ __launch_bounds__(256) void ec_lse_kernel(const float* __restrict__ logits, int64_t T,
                                                     int E, int64_t C, int S, int sigmoid,
                                                     float* __restrict__ norm,
                                                     int32_t* __restrict__ token_row,
                                                     int32_t* __restrict__ rows,
                                                     double* __restrict__ zpart) {
  __shared__ double red[256];
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  double z = 0.0;
  if (t < T) {
    const float* h = logits + t * E;
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, h[e]);
    float s = 0.f;
    for (int e = 0; e < E; ++e) s += expf(h[e] - m);
    const float l = m + logf(s);
    float ss = 0.f;
    if (sigmoid)
      for (int e = 0; e < E; ++e) ss += 1.0f / (1.0f + expf(-h[e]));
    norm[t] = sigmoid ? ss : l;
    z = (double)l * (double)l;
    for (int e = 0; e < E; ++e) token_row[t * E + e] = -1;
    if (S) rows[(int64_t)E * C + t] = (int32_t)t;
  }
  red[threadIdx.x] = z;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) zpart[blockIdx.x] = red[0];
}

// Block-wide exclusive prefix sum of one int per thread (256 threads, 4
// wavefronts): wave scans by shuffles, then the wave totals. Returns the prefix
// and writes the block total to *total.
template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += w < wave ? wave_tot[w] : 0;
    all += wave_tot[w];
  }
  *total = all;
  __syncthreads();   // wave_tot is reused by the next call
  return before + incl - v;
}

__device__ __forceinline__ float key_score(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u ^ 0x80000000u) : ~u);
}

constexpr int kEcLdsKeys = 16384;   // keys and lse of one expert kept in LDS (128 KB)

// One block per expert e: the C tokens with the largest key(logits[t][e]), ties
// to the lower token. The expert's keys are staged in LDS when T <= 16384 (else
// read from L2). An exact radix select over four 8-bit digits finds the C-th
// largest key K and how many tokens equal to K to take. Then each thread takes
// a contiguous range of tokens (norm staged in
// LDS with the keys): two block scans (of its count of keys equal to K, then of
// its count of taken tokens) place its chosen tokens in ascending order:
// tokens[e][i] = t, gates[e][i] = g[t][e], token_row[t][e] = e C + i,
// rows[e C + i] = t. It also writes P_e (mean over all tokens of p[t][e], or of
// s[t][e] / norm[t] for the sigmoid router; float64 tree) and the balance
// counts of expert e into stats.
constexpr int kEcSelectThreads = 1024;
__global__ __launch_bounds__(kEcSelectThreads) void ec_select_kernel(
    const float* __restrict__ logits, const float* __restrict__ lse, int64_t T, int E, int64_t C,
    int sigmoid, int32_t* __restrict__ tokens, float* __restrict__ gates, int32_t* __restrict__ token_row,
    int32_t* __restrict__ rows, moe_stats* __restrict__ stats) {
  __shared__ uint32_t keys[kEcLdsKeys];
  __shared__ float lse_s[kEcLdsKeys];
  constexpr int NT = kEcSelectThreads, NW = NT / 64;
  __shared__ int hist[256];
  __shared__ int wave_tot[NW];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  __shared__ double red[NT];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const bool in_lds = T <= kEcLdsKeys;
  auto key_at = [&](int64_t t) -> uint32_t {
    return in_lds ? keys[t] : score_key(logits[t * E + e]);
  };
  auto lse_at = [&](int64_t t) -> float { return in_lds ? lse_s[t] : lse[t]; };
  if (in_lds) {
    // eight loads in flight per thread
    for (int64_t t0 = 0; t0 < T; t0 += 8 * NT) {
      float v[8], l[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t t = t0 + u * NT + tid;
        v[u] = t < T ? logits[t * E + e] : 0.f;
        l[u] = t < T ? lse[t] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t t = t0 + u * NT + tid;
        if (t < T) {
          keys[t] = score_key(v[u]);
          lse_s[t] = l[u];
        }
      }
    }
  }
  uint32_t prefix = 0, mask = 0;
  int remaining = (int)C;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int64_t t = tid; t < T; t += NT) {
      const uint32_t u = key_at(t);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    // digits in descending order, thread i holding digit 255 - i: the digit D is
    // the one at which the running count of larger-or-equal digits first
    // reaches `remaining`
    // (threads past 256 hold no digit)
    const int dg = 255 - tid;
    const int cnt = tid < 256 ? hist[dg] : 0;
    int tot = 0;
    const int above = block_exclusive_scan<NW>(cnt, wave_tot, &tot);
    if (tid < 256 && above < remaining && above + cnt >= remaining) {
      s_prefix = prefix | ((uint32_t)dg << shift);
      s_remaining = remaining - above;
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 0xFFu << shift;
  }
  // prefix = K; remaining = tokens with key == K to take (lowest tokens first)
  const int64_t chunk = (T + NT - 1) / NT;
  const int64_t lo = tid * chunk < T ? tid * chunk : T;
  const int64_t hi = lo + chunk < T ? lo + chunk : T;
  int n_gt = 0, n_eq = 0;
  for (int64_t t = lo; t < hi; ++t) {
    const uint32_t u = key_at(t);
    n_gt += u > prefix;
    n_eq += u == prefix;
  }
  int tot = 0;
  const int eq_before = block_exclusive_scan<NW>(n_eq, wave_tot, &tot);
  int eq_take = remaining - eq_before;
  eq_take = eq_take < 0 ? 0 : (eq_take > n_eq ? n_eq : eq_take);
  const int pos0 = block_exclusive_scan<NW>(n_gt + eq_take, wave_tot, &tot);
  int pos = pos0, eq_seen = 0;
  double psum = 0.0;
  for (int64_t t = lo; t < hi; ++t) {
    const uint32_t u = key_at(t);
    const float h = key_score(u);
    float p, a;
    if (sigmoid) {
      p = 1.0f / (1.0f + expf(-h));
      a = p / lse_at(t);
    } else {
      p = expf(h - lse_at(t));
      a = p;
    }
    psum += (double)a;
    bool take = u > prefix;
    if (u == prefix) {
      take = eq_seen < eq_take;
      ++eq_seen;
    }
    if (take && pos < C) {
      const int64_t r = (int64_t)e * C + pos;
      tokens[r] = (int32_t)t;
      gates[r] = p;
      token_row[t * E + e] = (int32_t)r;
      rows[r] = (int32_t)t;
      ++pos;
    }
  }
  red[tid] = psum;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
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

// One block: group offsets (e C; the shared group after E C), the z-loss from
// the per-block partials of ec_lse_kernel (added in block order), L_aux from
// the P_i (= sum_i P_i, since every f_i = 1 / E), the unpicked-token count
// zeroed for ec_combine_kernel to add to, and the unused expert slots cleared.
__global__ __launch_bounds__(256) void ec_finalize_kernel(const double* __restrict__ zpart,
                                                          int nzpart, int64_t T, int E, int64_t C,
                                                          int S, int32_t* __restrict__ offsets,
                                                          moe_stats* __restrict__ stats) {
  __shared__ double red[256];
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
  for (int b = tid; b < nzpart; b += 256) z += zpart[b];
  red[tid] = z;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    double laux = 0.0;
    for (int e = 0; e < E; ++e) laux += (double)stats->prob_mean[e];
    stats->z_loss = (float)(red[0] / (double)T);
    stats->l_aux = (float)laux;   // E sum_i f_i P_i with f_i = 1 / E
    stats->capacity = (int32_t)C;
    stats->kept = (int32_t)((int64_t)E * C);
    stats->dropped = 0;
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
                                                         T_* __restrict__ y,
                                                         moe_stats* __restrict__ stats) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int64_t nrows = (int64_t)E * C;
  // tokens no expert chose are counted into stats->dropped (integer sum)
  bool picked = false;
  for (int e = lane; e < E; e += 64) picked |= token_row[t * E + e] >= 0;
  const uint64_t any_picked = __ballot(picked);   // every lane takes part in the ballot
  if (lane == 0 && any_picked == 0ull) atomicAdd(&stats->dropped, 1);
  // every lane runs every column step (the ballots and shuffles below need the
  // whole wavefront); lanes past d only skip their loads and stores
  for (int c0 = 0; c0 < d; c0 += 512) {
    const int c = c0 + lane * 8;
    const bool active = c < d;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // experts in ascending order, 64 at a time: lane e holds expert e0 + e's row
    // and gate; the picked rows are then read four at a time (loads in flight
    // together) and added in expert order
    for (int e0 = 0; e0 < E; e0 += 64) {
      int myr = -1;
      float myg = 0.f;
      if (e0 + lane < E) {
        const int r = token_row[t * E + e0 + lane];
        if (r >= 0 && r < nrows) {
          myr = r;
          myg = gates[r];
        }
      }
      uint64_t mask = __ballot(myr >= 0);
      while (mask) {
        int rr[4];
        float gg[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          rr[q] = -1;
          gg[q] = 0.f;
          if (mask) {
            const int e = __ffsll((unsigned long long)mask) - 1;
            mask &= mask - 1;
            rr[q] = __shfl(myr, e, 64);
            gg[q] = __shfl(myg, e, 64);
          }
        }
        float a[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (active && rr[q] >= 0) load8(y_perm + (int64_t)rr[q] * d + c, a[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (active && rr[q] >= 0) {
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = fmaf(gg[q], a[q][u], v[u]);
          }
        }
      }
    }
    if (!active) continue;
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
  L.zpart = take((size_t)((T + 255) / 256) * 8);
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
  const unsigned lb = (unsigned)((T + 255) / 256);
  double* zpart = (double*)(ws + L.zpart);
  const int sig = c.score_fn == MOE_SCORE_SIGMOID ? 1 : 0;
  hipLaunchKernelGGL(ec_lse_kernel, dim3(lb), dim3(256), 0, s, (const float*)lg, T, E, C, S, sig,
                     lse, r.token_row, rows, zpart);
  hipLaunchKernelGGL(ec_select_kernel, dim3(E), dim3(kEcSelectThreads), 0, s, (const float*)lg,
                     (const float*)lse, T, E, C, sig, r.tokens, r.gates, r.token_row, rows, stats);
  hipLaunchKernelGGL(ec_finalize_kernel, dim3(1), dim3(256), 0, s, (const double*)zpart, (int)lb,
                     T, E, C, S, off, stats);
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
                       (const int32_t*)r.token_row, (const float*)r.gates, T, d, E, C, S, (bf16*)y,
                       stats);
  else
    hipLaunchKernelGGL((ec_combine_kernel<float>), dim3(tb), dim3(256), 0, s, (const float*)yp,
                       (const int32_t*)r.token_row, (const float*)r.gates, T, d, E, C, S,
                       (float*)y, stats);
  return hipGetLastError();
}

}  // namespace moe
