// Router: gate logits, score function, top-k with renormalised gates, and the
// per-block partial sums of the balance statistics (P_i and logsumexp^2).
//
// MoE From Scratch to DeepSeek V3: token-choice formula h(x) = x W_g,
// p = Softmax(h), Gate = TopK(p); router softmax forced to float32; z-loss
// log^2(sum e^logit); V3 sigmoid scores with a selection-only bias b_i.
// MoE Training: Mixture of Experts, "Basic MoE Architecture" (gate nn.Linear
// with bias, softmax, topk, divide by the top-k sum) and "3. Load Balancing".
#include "moe_internal.h"

namespace moe {

// logits[t][e] = sum_c x[t][c] w[e][c] (+ b[e]). One wavefront takes 8 tokens
// and 8 experts at a time: lanes split d into 8-element slices (16-byte loads
// of bf16 x), so each router weight load serves 8 tokens, and every lane keeps
// 64 float32 partial sums, one per (token, expert). Those are summed over the
// 64 lanes by a reduce-scatter (6 exchange steps, each lane keeping half of
// its values), after which lane l holds the total of (token l / 8, expert
// l % 8). The summation order is fixed, so the result is deterministic.
template <typename XT, typename WT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const WT* __restrict__ wg,
                                                            const float* __restrict__ bg,
                                                            float* __restrict__ logits, int64_t T,
                                                            int d, int E) {
  const int lane = threadIdx.x & 63;
  const int64_t ngroups = (T + 7) / 8;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t tg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); tg < ngroups; tg += nwaves) {
    const int64_t t0 = tg * 8;
    for (int e0 = 0; e0 < E; e0 += 8) {
      const int ne = min(8, E - e0);
      float v[64];   // v[tok * 8 + e]
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = 0.f;
      for (int c = lane * 8; c < d; c += 512) {
        float wv[8][8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ee = e0 + min(e, ne - 1);   // missing experts repeat the last (not stored)
          load8(wg + (int64_t)ee * d + c, wv[e]);
        }
#pragma unroll
        for (int tk = 0; tk < 8; ++tk) {
          float xv[8];
          load8(x + min(t0 + tk, T - 1) * d + c, xv);
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int q = 0; q < 8; ++q) v[tk * 8 + e] = fmaf(xv[q], wv[e][q], v[tk * 8 + e]);
        }
      }
      // reduce-scatter over the wave: at the step with lane bit s, the lane
      // keeps the half of its n values selected by that bit and adds the
      // partner's copy of it
#pragma unroll
      for (int s2 = 32, n = 64; s2 >= 1; s2 >>= 1, n >>= 1) {
        const bool hi = (lane & s2) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
          const float send = hi ? v[i] : v[i + n / 2];
          const float keep = hi ? v[i + n / 2] : v[i];
          v[i] = keep + __shfl_xor(send, s2, 64);
        }
      }
      const int64_t t = t0 + (lane >> 3);
      const int e = e0 + (lane & 7);
      if (t < T && (lane & 7) < ne) logits[t * E + e] = bg ? v[0] + bg[e] : v[0];
    }
  }
}

// Butterfly exchange over groups of L lanes (L a power of two <= 64), level
// by level: lane i receives the value of its partner at levels 1 and 2 (DPP
// quad permutations, lanes i ^ 1 and i ^ 2), 4 (DPP mirror within 8 lanes,
// i ^ 7) and 8 (DPP mirror within 16 lanes, i ^ 15), then lanes i ^ 16 and
// i ^ 32 (LDS permute). The first four are plain ALU moves; after levels
// 1, 2, 4, 8, ... every lane of a group has combined all of the group's
// values, as with partners i ^ 1, i ^ 2, i ^ 4, i ^ 8. Every lane of the
// wave must be active.
template <int LVL>
__device__ __forceinline__ int lane_xchg(int v) {
  if constexpr (LVL == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  else if constexpr (LVL == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  else if constexpr (LVL == 4) return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
  else if constexpr (LVL == 8) return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
  else return __shfl_xor(v, LVL, 64);
}
template <int LVL>
__device__ __forceinline__ float lane_xchg(float v) {
  return __int_as_float(lane_xchg<LVL>(__float_as_int(v)));
}
template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L > 1) v = fmaxf(v, lane_xchg<1>(v));
  if constexpr (L > 2) v = fmaxf(v, lane_xchg<2>(v));
  if constexpr (L > 4) v = fmaxf(v, lane_xchg<4>(v));
  if constexpr (L > 8) v = fmaxf(v, lane_xchg<8>(v));
  if constexpr (L > 16) v = fmaxf(v, lane_xchg<16>(v));
  if constexpr (L > 32) v = fmaxf(v, lane_xchg<32>(v));
  return v;
}
// (every lane of a group ends with the same sum: each level adds two equal
// partial sums in either order)
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L > 1) v += lane_xchg<1>(v);
  if constexpr (L > 2) v += lane_xchg<2>(v);
  if constexpr (L > 4) v += lane_xchg<4>(v);
  if constexpr (L > 8) v += lane_xchg<8>(v);
  if constexpr (L > 16) v += lane_xchg<16>(v);
  if constexpr (L > 32) v += lane_xchg<32>(v);
  return v;
}

// (key, index) order used for selection: larger key first, then lower index.
// An out-of-range index (>= E) never beats an in-range one.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib, int E) {
  if (ia >= E) return false;
  if (ib >= E) return true;
  return ka > kb || (ka == kb && ia < ib);
}

// Score function + top-k + gates of one token, held by L lanes with J experts
// per lane (expert e = lane_in_group + L * jj, l[jj] its logit, -inf past E):
// writes the token's top-k when valid and adds its P contribution per expert
// to pacc and its lse^2 to lacc.
template <int L, int J>
__device__ __forceinline__ void route_token(const float l[J], bool valid, int64_t t, int lg, int tid,
                                            int E, int k, int sigmoid,
                                            const float* __restrict__ e_bias,
                                            int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_gate, float pacc[J],
                                            float& lacc) {
  float key[J], sc[J];
  bool taken[J];
  float m = -INFINITY;
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int e = lg + L * jj;
    taken[jj] = false;
    if (e < E) m = fmaxf(m, l[jj]);
  }
  m = group_max<L>(m);
  float ex[J];
  float s = 0.f;
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int e = lg + L * jj;
    ex[jj] = (e < E) ? expf(l[jj] - m) : 0.f;
    s += ex[jj];
  }
  s = group_sum<L>(s);
  const float lse = m + logf(s);
  float ssum = 0.f;
  if (!sigmoid) {
    const float inv = 1.0f / s;
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      sc[jj] = ex[jj] * inv;   // p
      key[jj] = l[jj];         // softmax is increasing: rank by logit
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const int e = lg + L * jj;
      if (e < E) {
        sc[jj] = 1.0f / (1.0f + expf(-l[jj]));
        key[jj] = e_bias ? sc[jj] + e_bias[e] : sc[jj];
      } else {
        sc[jj] = 0.f;
        key[jj] = -INFINITY;
      }
      ssum += sc[jj];
    }
    ssum = group_sum<L>(ssum);
  }

  int sel_idx[MOE_MAX_TOP_K];
  float sel_sc[MOE_MAX_TOP_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K; ++j) {
    sel_idx[j] = 0;
    sel_sc[j] = 0.f;
    if (j < k) {
      float bk = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int jj = 0; jj < J; ++jj) {
        const int e = lg + L * jj;
        if (e < E && !taken[jj] && better(key[jj], e, bk, bi, E)) {
          bk = key[jj];
          bi = e;
        }
      }
      // (key, index) maximum over the group, level by level
#define MOE_ARGMAX_LVL(LVL)                                                           \
  if constexpr (L > (LVL)) {                                                          \
    const float ok = lane_xchg<LVL>(bk);                                              \
    const int oi = lane_xchg<LVL>(bi);                                                \
    if (better(ok, oi, bk, bi, E)) {                                                  \
      bk = ok;                                                                        \
      bi = oi;                                                                        \
    }                                                                                 \
  }
      MOE_ARGMAX_LVL(1)
      MOE_ARGMAX_LVL(2)
      MOE_ARGMAX_LVL(4)
      MOE_ARGMAX_LVL(8)
      MOE_ARGMAX_LVL(16)
      MOE_ARGMAX_LVL(32)
#undef MOE_ARGMAX_LVL
      // bi is uniform over the group; fetch its score from the owning lane.
      const int owner_j = bi / L;
      float mine = 0.f;
#pragma unroll
      for (int jj = 0; jj < J; ++jj) {
        if (jj == owner_j) mine = sc[jj];
        if (jj == owner_j && lg == bi % L) taken[jj] = true;
      }
      sel_idx[j] = bi;
      sel_sc[j] = __shfl(mine, (tid & ~(L - 1) & 63) + bi % L, 64);
    }
  }
  float tsum = 0.f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K; ++j)
    if (j < k) tsum += sel_sc[j];
  const float tinv = 1.0f / tsum;
  if (valid) {
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOP_K; ++j) {
      if (j < k && lg == j) {
        topk_idx[t * k + j] = sel_idx[j];
        topk_gate[t * k + j] = sel_sc[j] * tinv;
      }
    }
    const float pinv = sigmoid ? 1.0f / ssum : 1.0f;
#pragma unroll
    for (int jj = 0; jj < J; ++jj) pacc[jj] += sc[jj] * pinv;
    lacc += lse * lse;
  }
}

// Score function + top-k + gates for L lanes per token, J experts per lane
// (expert e = lane_in_group + L * jj). Also accumulates, per block and in a
// fixed order, sum_t P-contribution per expert and sum_t lse_t^2.
template <int L, int J>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ e_bias, int64_t T, int E, int k,
    int sigmoid, int iters, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    float* __restrict__ partials) {
  constexpr int GPB = 256 / L;
  __shared__ float red[GPB * L * J];
  __shared__ float red2[GPB];
  const int tid = threadIdx.x;
  const int g = tid / L;
  const int lg = tid % L;
  float pacc[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) pacc[jj] = 0.f;
  float lacc = 0.f;

  for (int it = 0; it < iters; ++it) {
    const int64_t t = ((int64_t)blockIdx.x * iters + it) * GPB + g;
    const bool valid = t < T;
    float l[J];
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const int e = lg + L * jj;
      l[jj] = (e < E) ? (valid ? logits[t * E + e] : 0.f) : -INFINITY;
    }
    route_token<L, J>(l, valid, t, lg, tid, E, k, sigmoid, e_bias, topk_idx, topk_gate, pacc, lacc);
  }

#pragma unroll
  for (int jj = 0; jj < J; ++jj) red[g * L * J + jj * L + lg] = pacc[jj];
  if (lg == 0) red2[g] = lacc;
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float s = 0.f;
    for (int gg = 0; gg < GPB; ++gg) s += red[gg * L * J + e];
    partials[(int64_t)blockIdx.x * (E + 1) + e] = s;
  }
  if (tid == 0) {
    float s = 0.f;
    for (int gg = 0; gg < GPB; ++gg) s += red2[gg];
    partials[(int64_t)blockIdx.x * (E + 1) + E] = s;
  }
}

// logits on MFMA for up to 16 experts with bf16 x (v_mfma_f32_16x16x32_bf16,
// tokens as rows, experts as columns, experts past E held at zero weight).
// A float32 W_g enters as three bf16 planes, w = hi + mid + lo with hi the
// bf16 rounding of w, mid that of w - hi and lo that of the rest (all 24
// significand bits), so x w = x hi + x mid + x lo with every product exact
// in float32: the logits match a float32 dot product to within float32
// accumulation error. A bf16 W_g is one plane. One block takes 32 tokens and
// K in 1024-deep chunks: a chunk's x fragments (16 per lane) and W_g values
// (64 per thread: 8 experts x 2 adjacent k x 4 tiles of 256) are loaded at
// once, W_g is written to LDS as bf16 planes, and after one barrier wave w
// multiplies k in [64 w, 64 w + 64) of each 256-deep tile; the four waves'
// sums are added in wave order at the end.
// With LR > 0 the same block then routes its 32 tokens (route_token with LR
// lanes per token, on exactly the logits it stored) and writes its partial
// sums of P_i and lse^2, as router_topk_kernel does.
template <bool W_F32, int LR>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(
    const bf16* __restrict__ x, const void* __restrict__ wg, const float* __restrict__ bg,
    float* __restrict__ logits, int64_t T, int d, int E, const float* __restrict__ e_bias,
    int k, int sigmoid, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    float* __restrict__ partials) {
  constexpr int NP = W_F32 ? 3 : 1;
  constexpr int KC = 1024, ROW = KC + 8;   // padded LDS row (bf16)
  __shared__ bf16 wp[NP][16][ROW];
  __shared__ float red[4][32][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int e0 = (tid >> 7) * 8;      // this thread's 8 experts (staging)
  const int kp = (tid & 127) * 2;     // and its 2 adjacent k of each tile
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int64_t ta = min(t0 + r, T - 1), tb = min(t0 + 16 + r, T - 1);
  f32x4 acc[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) acc[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < d; kc += KC) {
    const int ntile = min(4, (d - kc) / 256);
    bf16x8 xa[4][2][2];
    float2 wv[4][8];
    // all loads are unconditional so that they issue back to back: tiles past
    // the chunk's end reload its last tile (never used), and experts past E
    // read row E - 1 and are zeroed after the load (a load under a branch
    // gets its own wait for every load in flight)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = kc + min(j, ntile - 1) * 256;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kk = kb + wave * 64 + s2 * 32 + kq * 8;
        xa[j][s2][0] = *reinterpret_cast<const bf16x8*>(x + ta * d + kk);
        xa[j][s2][1] = *reinterpret_cast<const bf16x8*>(x + tb * d + kk);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool live = e0 + e < E;
        const int64_t o = (int64_t)min(e0 + e, E - 1) * d + kb + kp;
        if constexpr (W_F32) {
          const float2 w = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(wg) + o);
          wv[j][e] = make_float2(live ? w.x : 0.f, live ? w.y : 0.f);
        } else {
          uint32_t u = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const bf16*>(wg) + o);
          u = live ? u : 0u;
          wv[j][e] = make_float2(bf16_bits_to_f32(u & 0xffffu), bf16_bits_to_f32(u >> 16));
        }
      }
    }
    if (kc > 0) __syncthreads();   // the previous chunk's planes have been read
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < ntile) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 w = wv[j][e];
          const uint32_t hq = pack_bf16x2(w.x, w.y);
          *reinterpret_cast<uint32_t*>(&wp[0][e0 + e][j * 256 + kp]) = hq;
          if constexpr (W_F32) {
            const float hx = bf16_bits_to_f32(hq & 0xffffu), hy = bf16_bits_to_f32(hq >> 16);
            const float rx = w.x - hx, ry = w.y - hy;
            const uint32_t mq = pack_bf16x2(rx, ry);
            *reinterpret_cast<uint32_t*>(&wp[1][e0 + e][j * 256 + kp]) = mq;
            *reinterpret_cast<uint32_t*>(&wp[2][e0 + e][j * 256 + kp]) =
                pack_bf16x2(rx - bf16_bits_to_f32(mq & 0xffffu), ry - bf16_bits_to_f32(mq >> 16));
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < ntile) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int kk = j * 256 + wave * 64 + s2 * 32 + kq * 8;
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) {
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(&wp[pl][r][kk]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
              acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j][s2][m], b, acc[m], 0, 0, 0);
          }
        }
      }
    }
  }
  // element i of lane l holds token 4 (l / 16) + i and expert l % 16 of a subtile
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][m * 16 + 4 * kq + i][r] = acc[m][i];
  __syncthreads();
#pragma unroll
  for (int o = tid; o < 32 * 16; o += 256) {
    const int tt = o >> 4, e = o & 15;
    const int64_t t = t0 + tt;
    if (e < E && t < T) {
      const float v = ((red[0][tt][e] + red[1][tt][e]) + red[2][tt][e]) + red[3][tt][e];
      logits[t * E + e] = bg ? v + bg[e] : v;
    }
  }
  if constexpr (LR > 0) {
    constexpr int TPP = 256 / LR;   // tokens per pass
    __shared__ float rp[256], rl[256];
    const int lg = tid % LR;
    float pacc[1] = {0.f};
    float lacc = 0.f;
#pragma unroll
    for (int tt0 = 0; tt0 < 32; tt0 += TPP) {
      const int tt = tt0 + tid / LR;
      const int64_t t = t0 + tt;
      const bool valid = tt < 32 && t < T;
      float l[1];
      l[0] = -INFINITY;
      if (lg < E) {
        l[0] = 0.f;
        if (valid) {
          const float v = ((red[0][tt][lg] + red[1][tt][lg]) + red[2][tt][lg]) + red[3][tt][lg];
          l[0] = bg ? v + bg[lg] : v;
        }
      }
      route_token<LR, 1>(l, valid, t, lg, tid, E, k, sigmoid, e_bias, topk_idx, topk_gate, pacc,
                         lacc);
    }
    rp[tid] = pacc[0];
    rl[tid] = lacc;
    __syncthreads();
    if (tid < E) {
      float sum = 0.f;
      for (int g = 0; g < TPP; ++g) sum += rp[g * LR + tid];
      partials[(int64_t)blockIdx.x * (E + 1) + tid] = sum;
    }
    if (tid == 0) {
      float sum = 0.f;
      for (int g = 0; g < TPP; ++g) sum += rl[g * LR];
      partials[(int64_t)blockIdx.x * (E + 1) + E] = sum;
    }
  }
}

// P_i = (1/T) sum of the per-block partials and z = (1/T) sum_t lse_t^2:
// block e < E reduces column e, block E the lse^2 column, and block E + 1
// zero-fills the unused expert slots (route_stats_column).
__global__ __launch_bounds__(256) void route_stats_kernel(const float* __restrict__ partials,
                                                          int nblocks, int E, int64_t T,
                                                          moe_stats* __restrict__ stats) {
  __shared__ double red[256];
  route_stats_column(partials, nblocks, E, T, stats, (int)blockIdx.x, red);
}

template <int L, int J>
static void launch_topk_lj(const moe_config& c, const WsLayout& Lw, const float* logits,
                           const float* e_bias, int32_t* idx, float* gate, float* partials,
                           hipStream_t s) {
  hipLaunchKernelGGL((router_topk_kernel<L, J>), dim3(Lw.route_blocks), dim3(256), 0, s, logits,
                     e_bias, (int64_t)c.tokens, c.num_experts, c.top_k,
                     c.score_fn == MOE_SCORE_SIGMOID ? 1 : 0, Lw.route_iters, idx, gate, partials);
}

int route_lanes(int E) {
  int L = 1;
  while (L < E && L < 64) L <<= 1;
  return L;
}

// The MFMA logits kernel for a few experts (bf16 x, at most 16 experts).
static bool router_mfma_small(const moe_config& c) {
  return router_kparts(c) == 0 && c.act_dtype == MOE_BF16 && c.num_experts <= 16 &&
         c.d_model % 256 == 0;
}

template <bool W_F32, int LR>
static void launch_route_fused(const moe_config& c, const void* x, const void* w_gate,
                               const float* bg, float* lg, const float* eb, int32_t* idx,
                               float* gate, float* partials, hipStream_t s) {
  const unsigned mblocks = (unsigned)((c.tokens + 31) / 32);
  hipLaunchKernelGGL((router_logits_mfma_kernel<W_F32, LR>), dim3(mblocks), dim3(256), 0, s,
                     (const bf16*)x, w_gate, bg, lg, (int64_t)c.tokens, (int)c.d_model,
                     c.num_experts, eb, c.top_k, c.score_fn == MOE_SCORE_SIGMOID ? 1 : 0, idx,
                     gate, partials);
}

hipError_t launch_router_logits(const moe_config& c, const void* x, const void* w_gate,
                                const float* b_gate, float* lg, float* router_planes,
                                hipStream_t s) {
  const int E = c.num_experts;
  const int d = (int)c.d_model;
  const float* bg = c.has_gate_bias ? b_gate : nullptr;
  const int64_t waves = (c.tokens + 7) / 8;   // one wave per 8 tokens
  const int blocks = (int)((waves + 3) / 4 < 4096 ? (waves + 3) / 4 : 4096);
  if (router_kparts(c) > 0)
    return launch_router_gemm(c, x, w_gate, bg, router_planes, lg, s);
  if (router_mfma_small(c)) {
    const unsigned mblocks = (unsigned)((c.tokens + 31) / 32);
    if (c.router_dtype == MOE_F32)
      hipLaunchKernelGGL((router_logits_mfma_kernel<true, 0>), dim3(mblocks), dim3(256), 0, s,
                         (const bf16*)x, w_gate, bg, lg, (int64_t)c.tokens, d, E, nullptr, 0, 0,
                         nullptr, nullptr, nullptr);
    else
      hipLaunchKernelGGL((router_logits_mfma_kernel<false, 0>), dim3(mblocks), dim3(256), 0, s,
                         (const bf16*)x, w_gate, bg, lg, (int64_t)c.tokens, d, E, nullptr, 0, 0,
                         nullptr, nullptr, nullptr);
  } else if (c.act_dtype == MOE_BF16 && c.router_dtype == MOE_F32)
    hipLaunchKernelGGL((router_logits_kernel<bf16, float>), dim3(blocks), dim3(256), 0, s,
                       (const bf16*)x, (const float*)w_gate, bg, lg, (int64_t)c.tokens, d, E);
  else if (c.act_dtype == MOE_BF16)
    hipLaunchKernelGGL((router_logits_kernel<bf16, bf16>), dim3(blocks), dim3(256), 0, s,
                       (const bf16*)x, (const bf16*)w_gate, bg, lg, (int64_t)c.tokens, d, E);
  else if (c.router_dtype == MOE_F32)
    hipLaunchKernelGGL((router_logits_kernel<float, float>), dim3(blocks), dim3(256), 0, s,
                       (const float*)x, (const float*)w_gate, bg, lg, (int64_t)c.tokens, d, E);
  else
    hipLaunchKernelGGL((router_logits_kernel<float, bf16>), dim3(blocks), dim3(256), 0, s,
                       (const float*)x, (const bf16*)w_gate, bg, lg, (int64_t)c.tokens, d, E);
  return hipGetLastError();
}

hipError_t launch_route(const moe_config& c, const WsLayout& L, const void* x, const void* w_gate,
                        const float* b_gate, const float* e_bias, float* logits, int32_t* topk_idx,
                        float* topk_gate, moe_stats* stats, char* ws, hipStream_t s,
                        int* defer_stats) {
  const int E = c.num_experts;
  float* lg = logits ? logits : reinterpret_cast<float*>(ws + L.logits);
  float* partials = reinterpret_cast<float*>(ws + L.route_partials);
  const float* eb = c.score_fn == MOE_SCORE_SIGMOID ? e_bias : nullptr;
  const int Ln = route_lanes(E);
  if (router_mfma_small(c)) {
    // logits, top-k and the block partials in one kernel
    const float* bg = c.has_gate_bias ? b_gate : nullptr;
    const bool f32w = c.router_dtype == MOE_F32;
    switch (Ln) {
      case 1: f32w ? launch_route_fused<true, 1>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s)
                   : launch_route_fused<false, 1>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s); break;
      case 2: f32w ? launch_route_fused<true, 2>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s)
                   : launch_route_fused<false, 2>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s); break;
      case 4: f32w ? launch_route_fused<true, 4>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s)
                   : launch_route_fused<false, 4>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s); break;
      case 8: f32w ? launch_route_fused<true, 8>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s)
                   : launch_route_fused<false, 8>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s); break;
      default: f32w ? launch_route_fused<true, 16>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s)
                    : launch_route_fused<false, 16>(c, x, w_gate, bg, lg, eb, topk_idx, topk_gate, partials, s);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int pb = (int)((c.tokens + 31) / 32);
    if (defer_stats) {
      *defer_stats = pb;
      return hipSuccess;
    }
    hipLaunchKernelGGL(route_stats_kernel, dim3(E + 2), dim3(256), 0, s, partials, pb, E,
                       (int64_t)c.tokens, stats);
    return hipGetLastError();
  }
  hipError_t err = launch_router_logits(c, x, w_gate, b_gate, lg,
                                        reinterpret_cast<float*>(ws + L.router_planes), s);
  if (err != hipSuccess) return err;

  switch (Ln) {
    case 1: launch_topk_lj<1, 1>(c, L, lg, eb, topk_idx, topk_gate, partials, s); break;
    case 2: launch_topk_lj<2, 1>(c, L, lg, eb, topk_idx, topk_gate, partials, s); break;
    case 4: launch_topk_lj<4, 1>(c, L, lg, eb, topk_idx, topk_gate, partials, s); break;
    case 8: launch_topk_lj<8, 1>(c, L, lg, eb, topk_idx, topk_gate, partials, s); break;
    case 16: launch_topk_lj<16, 1>(c, L, lg, eb, topk_idx, topk_gate, partials, s); break;
    case 32: launch_topk_lj<32, 1>(c, L, lg, eb, topk_idx, topk_gate, partials, s); break;
    default: {
      const int J = (E + 63) / 64;
      if (J == 1) launch_topk_lj<64, 1>(c, L, lg, eb, topk_idx, topk_gate, partials, s);
      else if (J == 2) launch_topk_lj<64, 2>(c, L, lg, eb, topk_idx, topk_gate, partials, s);
      else if (J == 3) launch_topk_lj<64, 3>(c, L, lg, eb, topk_idx, topk_gate, partials, s);
      else launch_topk_lj<64, 4>(c, L, lg, eb, topk_idx, topk_gate, partials, s);
    }
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (defer_stats) {
    *defer_stats = L.route_blocks;
    return hipSuccess;
  }
  hipLaunchKernelGGL(route_stats_kernel, dim3(E + 2), dim3(256), 0, s, partials,
                     L.route_blocks, E, (int64_t)c.tokens, stats);
  return hipGetLastError();
}

}  // namespace moe
