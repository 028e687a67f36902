// Backward pass of the MoE layer (bf16 activations, float32 router and
// gradients), and the activation step of the training forward that saves the
// pre-activation. The grouped GEMMs of the backward are in expert_gemm.hip;
// these are the memory-bound steps around them.
//
// Objective differentiated: L = <dy, y> + aux_coef L_aux + z_coef z, with the
// forward of "MoE From Scratch to DeepSeek V3" (token-choice top-k, gate
// renormalisation, auxiliary loss, router z-loss, sigmoid routing with a
// selection bias, shared experts) and the expert FFN of "MoE Training: Mixture
// of Experts" ("Basic MoE Architecture"). Top-k choices, capacity decisions and
// the counts f_i carry no gradient; the selection bias receives none.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ float act_bf16(int act, float z) {
  return act == MOE_ACT_GELU ? gelu_poly(z) : fmaxf(z, 0.f);
}

// SwiGLU on the saved planes: h = silu(z1) u.
__device__ __forceinline__ float swiglu_h(float z1, float u) { return silu(z1) * u; }

__device__ __forceinline__ int clamp_off(const int32_t* __restrict__ off, int g, int64_t rows_max) {
  const int v = off[g];
  return v < 0 ? 0 : (v > rows_max ? (int)rows_max : v);
}

// ------------------------------------------------------------------ training forward
// h[r] = act(z[r]) for the rows r < expert_offsets[G] (z already rounded to
// bf16, so the backward recomputes exactly this h); SwiGLU: h = silu(z1) u with
// u the second plane (u != nullptr). 8 elements per thread.
__global__ __launch_bounds__(256) void act_rows_kernel(const bf16* __restrict__ z,
                                                       const bf16* __restrict__ u,
                                                       const int32_t* __restrict__ off, int G,
                                                       int64_t rows_max, int F, int act,
                                                       bf16* __restrict__ h) {
  const int64_t R = clamp_off(off, G, rows_max);
  const int64_t n8 = R * F / 8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    load8(z + i * 8, v);
    if (u) {
      float w[8];
      load8(u + i * 8, w);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = swiglu_h(v[e], w[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = act_bf16(act, v[e]);
    }
    store8(h + i * 8, v);
  }
}

// SwiGLU backward, elementwise: from dH, z1 and u (rows r < expert_offsets[G]),
// dz1 = dH u silu'(z1) and du = dH silu(z1), written side by side as row r of
// dZ [rows][2F] (dz1 in columns 0..F-1, du in F..2F-1).
__global__ __launch_bounds__(256) void dswiglu_kernel(const bf16* __restrict__ dh,
                                                      const bf16* __restrict__ z1,
                                                      const bf16* __restrict__ u,
                                                      const int32_t* __restrict__ off, int G,
                                                      int64_t rows_max, int F,
                                                      bf16* __restrict__ dz) {
  const int64_t R = clamp_off(off, G, rows_max);
  const int64_t n8 = R * F / 8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i * 8 / F, c = i * 8 - r * F;
    float g[8], a[8], b[8], o1[8], o2[8];
    load8(dh + i * 8, g);
    load8(z1 + i * 8, a);
    load8(u + i * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sg = 1.0f / (1.0f + expf(-a[e]));
      const float si = a[e] * sg;
      o1[e] = g[e] * b[e] * sg * (1.0f + a[e] * (1.0f - sg));
      o2[e] = g[e] * si;
    }
    store8(dz + r * 2 * F + c, o1);
    store8(dz + r * 2 * F + F + c, o2);
  }
}

// ------------------------------------------------------------------ combine backward
// One wavefront per token t. For each choice j with row r = assign_row[t, j]
// (kept): dYp[r] = g[t, j] dy[t] (bf16) and dgate[t, j] = <dy[t], y_perm[r]>
// (float32, lanes then a wave reduction); dropped choices get dgate = 0. With a
// shared expert, its row expert_offsets[E] + t receives dy[t] (gate 1).
// ET: the layer's activation type (bf16, or float for float32 layers).
template <typename ET>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const ET* __restrict__ dy, const ET* __restrict__ y_perm, const float* __restrict__ gate,
    const int32_t* __restrict__ assign_row, const int32_t* __restrict__ off, int64_t T, int d, int k,
    int E, int S, int64_t rows_max, ET* __restrict__ dyp, float* __restrict__ dgate) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const ET* dyt = dy + t * d;
  for (int j = 0; j < k; ++j) {
    const int r = assign_row[t * k + j];
    float dot = 0.f;
    if (r >= 0 && r < rows_max) {
      const float g = gate[t * k + j];
      const ET* yr = y_perm + (int64_t)r * d;
      ET* out = dyp + (int64_t)r * d;
      for (int c = lane * 8; c < d; c += 512) {
        float a[8], b[8];
        load8(dyt + c, a);
        load8(yr + c, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dot = fmaf(a[e], b[e], dot);
          a[e] *= g;
        }
        store8(out + c, a);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
    if (lane == 0) dgate[t * k + j] = dot;
  }
  if (S) {
    const int64_t r = (int64_t)clamp_off(off, E, rows_max) + t;
    if (r < rows_max) {
      ET* out = dyp + r * d;
      for (int c = lane * 8; c < d; c += 512) {
        float a[8];
        load8(dyt + c, a);
        store8(out + c, a);
      }
    }
  }
}

// ------------------------------------------------------------------ router backward
// W lanes per token (W = the power of two >= E, at most 64; 64 / W tokens per
// wavefront); lane l of a token's W holds experts l, l + 64, l + 128, l + 192
// (only l when E <= 64). The reductions over a token's lanes are xor trees of
// width W, which add the same terms in the same order as a 64-wide tree over
// the zero-padded row.
// Gates g_j = s_{i_j} / S (S = sum of the selected scores) give
// ds_{i_j} = (dg_j - sum_m dg_m g_m) / S; L_aux = E sum_i f_i P_i adds
// dq_i = aux_coef E f_i / T to the probabilities it averages (softmax: p;
// sigmoid: q = s / sum s, taken back through the normalisation); then the
// softmax Jacobian p (ds - <ds, p>) or the sigmoid derivative s (1 - s), and
// the z-loss term z_coef 2 lse p / T. float32 throughout (the router's
// precision).
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dgate, const int32_t* __restrict__ counts_pre, int64_t T, int E,
    int k, int sigmoid, float aux_coef, float z_coef, float* __restrict__ dlogits) {
  const int W = E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64));
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / W;
  const int lane = threadIdx.x & (W - 1);
  if (t >= T) return;
  const float* h = logits + t * E;
  float hv[4];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    hv[i] = e < E ? h[e] : -INFINITY;
    m = fmaxf(m, hv[i]);
  }
#pragma unroll
  for (int o = W >> 1; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float se = 0.f;
  float ex[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ex[i] = lane + 64 * i < E ? expf(hv[i] - m) : 0.f;
    se += ex[i];
  }
#pragma unroll
  for (int o = W >> 1; o > 0; o >>= 1) se += __shfl_xor(se, o, 64);
  const float lse = m + logf(se);
  const float inv_se = 1.0f / se;
  // selected scores and the renormalised gates
  float ssel[MOE_MAX_TOP_K], dg[MOE_MAX_TOP_K];
  int isel[MOE_MAX_TOP_K];
  float S = 0.f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K; ++j) {
    isel[j] = -1;
    ssel[j] = dg[j] = 0.f;
    if (j < k) {
      int e = topk_idx[t * k + j];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      isel[j] = e;
      const float he = h[e];
      ssel[j] = sigmoid ? 1.0f / (1.0f + expf(-he)) : expf(he - m) * inv_se;
      dg[j] = dgate[t * k + j];
      S += ssel[j];
    }
  }
  float c0 = 0.f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K; ++j) c0 += dg[j] * (ssel[j] / S);
  const float aux_scale = aux_coef * (float)E / ((float)T * (float)T * (float)k);
  float p[4], s[4], ds[4], dq[4];
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    p[i] = ex[i] * inv_se;
    s[i] = e < E ? (sigmoid ? 1.0f / (1.0f + expf(-hv[i])) : p[i]) : 0.f;
    tot += s[i];
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOP_K; ++j) v += isel[j] == e ? (dg[j] - c0) / S : 0.f;
    ds[i] = v;
    dq[i] = e < E ? aux_scale * (float)counts_pre[e] : 0.f;   // aux_coef E f_e / T
  }
  float dh[4];
  if (!sigmoid) {
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ds[i] += dq[i];
      dot += ds[i] * p[i];
    }
#pragma unroll
    for (int o = W >> 1; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dh[i] = p[i] * (ds[i] - dot);
  } else {
#pragma unroll
    for (int o = W >> 1; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
    float dotq = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) dotq += dq[i] * (s[i] / tot);
#pragma unroll
    for (int o = W >> 1; o > 0; o >>= 1) dotq += __shfl_xor(dotq, o, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ds[i] += (dq[i] - dotq) / tot;
      dh[i] = ds[i] * s[i] * (1.0f - s[i]);
    }
  }
  const float zs = z_coef * 2.0f * lse / (float)T;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (e < E) dlogits[t * E + e] = fmaf(zs, p[i], dh[i]);
  }
}

// ------------------------------------------------------------------ weight and bias gradients
// so[g]: expert_offsets clamped to [0, rows_max] and made non-decreasing (a
// running maximum), so the groups' rows never sum past rows_max; po[g] = sum
// over g' < g of the padded row count of group g' (its rows rounded up to a
// multiple of 128, at least 128), hence po[G] <= rows_max + 128 G. One wave:
// lane l takes groups 5 l .. 5 l + 4 (G <= 257), then a prefix maximum and a
// prefix sum over the lanes.
__global__ __launch_bounds__(64) void pad_offsets_kernel(const int32_t* __restrict__ off, int G,
                                                         int64_t rows_max, int32_t* __restrict__ po,
                                                         int32_t* __restrict__ so) {
  constexpr int PER = 5;
  const int lane = threadIdx.x;
  if (blockIdx.x != 0 || lane >= 64) return;
  const int base = clamp_off(off, 0, rows_max);
  int hi[PER];
  int m = base;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = lane * PER + i;
    const int v = g < G ? clamp_off(off, g + 1, rows_max) : base;
    m = v > m ? v : m;
    hi[i] = m;
  }
  int incl = m;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl = t > incl ? t : incl;
  }
  const int up = __shfl_up(incl, 1, 64);
  const int before = lane == 0 ? base : up;   // so of this lane's first group
  int prev = before, sum = 0;
  int pad[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = lane * PER + i;
    const int h = hi[i] > before ? hi[i] : before;
    const int r = h - prev;
    pad[i] = g < G ? (r <= 128 ? 128 : (r + 127) & ~127) : 0;
    sum += pad[i];
    hi[i] = h;
    prev = h;
  }
  int isum = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(isum, o, 64);
    if (lane >= o) isum += t;
  }
  int acc = isum - sum;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = lane * PER + i;
    acc += pad[i];
    if (g < G) {
      po[g + 1] = acc;
      so[g + 1] = hi[i];
    }
  }
  if (lane == 0) {
    po[0] = 0;
    so[0] = base;
  }
}

// xp[r] = x[row_token[r]] for the kept rows r < so[G] (the expert-sorted copy of
// the token rows that the weight gradient of W1 / W3 reads; row_token clamped to
// [0, T)). 16 bytes per thread.
__global__ __launch_bounds__(256) void gather_rows_kernel(const bf16* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ so, int G,
                                                          int64_t T, int d, bf16* __restrict__ xp) {
  const int64_t R = so[G];
  const int c8 = d / 8;
  const int64_t n = R * c8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / c8;
    const int c = (int)(i - r * c8) * 8;
    int64_t t = row_token[r];
    t = t < 0 ? 0 : (t >= T ? T - 1 : t);
    *reinterpret_cast<uint4*>(xp + r * d + c) = *reinterpret_cast<const uint4*>(x + t * d + c);
  }
}

// Column sums of the expert-sorted rows of src ([rows][ld], columns 0..C-1)
// for the bias gradients, in blocks of 64 rows of the padded row space (so and
// po as written by pad_offsets_kernel): block (kb, cs) adds the rows
// so[g] + k - po[g] of its group g for k in [64 kb, 64 kb + 64) that lie inside
// the group, over columns 512 cs .. + 511, and writes partial[kb][c]. Thread:
// 8 columns, one of 4 row lanes (16 rows each, in order); the 4 lanes are then
// added in order (deterministic).
__global__ __launch_bounds__(256) void colsum_rows_kernel(const bf16* __restrict__ src, int ld,
                                                          int C, const int32_t* __restrict__ so,
                                                          const int32_t* __restrict__ po, int G,
                                                          float* __restrict__ partial) {
  __shared__ float red[4][512];
  const int k0 = blockIdx.x * 64;
  if (k0 >= po[G]) return;
  int lo = 0, hi = G;   // group of row k0: po[lo] <= k0 < po[lo + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (po[mid] <= k0) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int local = k0 - po[g];
  const int nr = so[g + 1] - so[g];
  const int rl = threadIdx.x >> 6;
  const int cl = (threadIdx.x & 63) * 8;
  const int c = blockIdx.y * 512 + cl;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c < C && local < nr) {
    // the 16 rows' loads issued together (rows past the group re-read its last
    // row and are not added)
    float v[16][8];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int lr = min(local + rl * 16 + j, nr - 1);
      load8(src + (int64_t)(so[g] + lr) * ld + c, v[j]);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool in = local + rl * 16 + j < nr;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += in ? v[j][e] : 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rl][cl + e] = acc[e];
  __syncthreads();
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cc = t + 256 * h;
    const int col = blockIdx.y * 512 + cc;
    if (col < C)
      partial[(int64_t)blockIdx.x * C + col] = ((red[0][cc] + red[1][cc]) + red[2][cc]) + red[3][cc];
  }
}

// db[g][c] = sum of the column sums of group g's 128-row M tiles (written by
// the dZ GEMM), in tile order. Group g's tiles follow those of the groups
// before it, ceil(rows / 128) tiles for a group of rows = o[g + 1] - o[g] > 0
// (o: offsets clamped to [0, rows_max]), as the GEMM's tile space counts them;
// tiles past cap (the partial buffer: only with malformed offsets) are left
// out. Routed groups write db + g C, the shared expert (g == E) writes dbs.
__global__ __launch_bounds__(256) void colsum_tiles_reduce_kernel(
    const float* __restrict__ partial, const int32_t* __restrict__ off, int G, int E,
    int64_t rows_max, int C, int cap, float* __restrict__ db, float* __restrict__ dbs) {
  __shared__ int s_tiles[MOE_MAX_EXPERTS + 1];
  __shared__ int s_first, s_n;
  const int g = blockIdx.y;
  for (int gi = threadIdx.x; gi < G; gi += blockDim.x) {
    const int a = clamp_off(off, gi, rows_max), b = clamp_off(off, gi + 1, rows_max);
    s_tiles[gi] = b > a ? (b - a + 127) / 128 : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int first = 0;
    for (int gi = 0; gi < g; ++gi) first += s_tiles[gi];
    s_first = first;
    s_n = s_tiles[g];
  }
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int first = s_first;
  const int n = first + s_n <= cap ? s_n : (first < cap ? cap - first : 0);
  float acc = 0.f;
  int i = 0;
  for (; i + 8 <= n; i += 8) {   // eight loads in flight, added in tile order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[(int64_t)(first + i + u) * C + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; i < n; ++i) acc += partial[(int64_t)(first + i) * C + c];
  if (g < E) db[(int64_t)g * C + c] = acc;
  else dbs[c] = acc;
}

// db[g][c] = sum of the column-sum partials of group g's 64-row blocks, in
// block order (deterministic). Routed groups write db + g C, the shared expert
// (g == E) writes dbs.
__global__ __launch_bounds__(256) void colsum_reduce_kernel(const float* __restrict__ partial,
                                                            int ldp, const int32_t* __restrict__ po,
                                                            int C, int E, float* __restrict__ db,
                                                            float* __restrict__ dbs) {
  const int g = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int b0 = po[g] / 64, b1 = po[g + 1] / 64;   // b1 - b0 is even (po: multiples of 128)
  float s = 0.f;
  int b = b0;
  for (; b + 8 <= b1; b += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[(int64_t)(b + u) * ldp + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; b < b1; ++b) s += partial[(int64_t)b * ldp + c];
  if (g < E) db[(int64_t)g * C + c] = s;
  else dbs[c] = s;
}

// ------------------------------------------------------------------ router weights
// dW_g[e][c] = sum_t dlogits[t][e] x[t][c]. Block (8 experts, 512 columns, a
// token slice); wave w takes the slice's tokens w, w + 4, w + 8, ..., lane =
// 8 consecutive columns (one 16-byte load per token) x 8 experts. Waves 1..3
// hand their sums to wave 0 through LDS, which adds them in wave order and
// writes partial[slice][e][c]; gate_wgrad_reduce_kernel adds the slices in
// order (deterministic).
__global__ __launch_bounds__(256) void gate_wgrad_kernel(const bf16* __restrict__ x,
                                                         const float* __restrict__ dlogits,
                                                         int64_t T, int d, int E, int slice_len,
                                                         float* __restrict__ partial) {
  __shared__ float red[3][64][65];
  const int e0 = blockIdx.x * 8;
  // the wave index is uniform: the token rows of dlogits are read with scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = (blockIdx.y * 64 + lane) * 8;
  const int64_t t0 = (int64_t)blockIdx.z * slice_len;
  const int64_t t1 = t0 + slice_len < T ? t0 + slice_len : T;
  float acc[8][8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[e][u] = 0.f;
  if (c < d) {
    // eight tokens per iteration, their loads issued together (tokens past the
    // slice re-read its last token and are not added)
    for (int64_t tb = t0 + wave; tb < t1; tb += 32) {
      float xv[8][8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t t = min(tb + 4 * q, t1 - 1);
        load8(x + t * d + c, xv[q]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t t = tb + 4 * q;
        if (t < t1) {
          const float* dl = dlogits + t * E + e0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float g = e0 + e < E ? dl[e] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[e][u] = fmaf(g, xv[q][u], acc[e][u]);
          }
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int u = 0; u < 8; ++u) red[wave - 1][lane][e * 8 + u] = acc[e][u];
  }
  __syncthreads();
  if (wave == 0 && c < d) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e0 + e < E) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = ((acc[e][u] + red[0][lane][e * 8 + u]) + red[1][lane][e * 8 + u]) +
                 red[2][lane][e * 8 + u];
        store8(partial + ((int64_t)blockIdx.z * E + e0 + e) * d + c, v);
      }
    }
  }
}

// dw[i] = sum over the slices of partial[slice][i], in slice order: block = 64
// outputs x 4 slice lanes (lane q adds slices [q S', (q + 1) S') in order,
// S' = ceil(slices / 4)), the lanes' sums then added in lane order.
__global__ __launch_bounds__(256) void gate_wgrad_reduce_kernel(const float* __restrict__ partial,
                                                                int slices, int64_t n,
                                                                float* __restrict__ dw) {
  __shared__ float red[4][64];
  const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t i = blockIdx.x * (int64_t)64 + lane;
  const int per = (slices + 3) / 4;
  const int z0 = q * per;
  const int z1 = z0 + per < slices ? z0 + per : slices;
  float s = 0.f;
  if (i < n) {
    int z = z0;
    for (; z + 8 <= z1; z += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = partial[(z + u) * n + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; z < z1; ++z) s += partial[z * n + i];
  }
  red[q][lane] = s;
  __syncthreads();
  if (q == 0 && i < n) dw[i] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// db_g[e] = sum_t dlogits[t][e]: one block per expert, a fixed-order tree.
__global__ __launch_bounds__(256) void gate_bias_grad_kernel(const float* __restrict__ dlogits,
                                                             int64_t T, int E,
                                                             float* __restrict__ db) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float s = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += 256) s += dlogits[t * E + e];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) db[e] = red[0];
}

// dlogits [T][E] float32 as two bf16 planes, dlp[t][e] = hi = bf16(v) and
// dlp[t][E + e] = lo = bf16(v - hi) (v - hi is exact; hi + lo = v to within
// 2^-17 |v|), so that a bf16 GEMM with float32 accumulation multiplies v by a
// bf16 operand with the products exact; block 0 also writes the bounds of
// `slices` equal token slices, gso[i] = i T / slices.
__global__ __launch_bounds__(256) void dlogit_planes_kernel(const float* __restrict__ dl, int64_t T,
                                                            int E, int slices,
                                                            bf16* __restrict__ dlp,
                                                            int32_t* __restrict__ gso) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && (int)threadIdx.x <= slices)
    gso[threadIdx.x] = (int32_t)(T * (int64_t)threadIdx.x / slices);
  if (i >= T * E) return;
  const int64_t t = i / E;
  const int e = (int)(i - t * E);
  const float v = dl[i];
  const bf16 hi = (bf16)v;
  dlp[t * 2 * E + e] = hi;
  dlp[t * 2 * E + E + e] = (bf16)(v - (float)hi);
}

// ------------------------------------------------------------------ dx
// dx[t] = sum_j dXp[assign_row[t, j]] (kept choices, j order) + dXp[off[E] + t]
// (shared expert) + sum_e dlogits[t][e] W_g[e] (router), float32 sums, one
// rounding. One wavefront per token; lanes take 16-byte column chunks.
// KM >= k bounds the row slots at compile time. Loads are unconditional so a
// lane's loads issue before the first use (a load under a branch gets a wait
// of its own): W_g rows in batches of 8 (rows past E reread row E - 1), and
// row slots that are dropped or past k reread the token's first live row; all
// of them are masked out of the sums, which keep the order above.
// With xr, the router term is read from xr [T][d] (computed on MFMA) instead.
template <typename ET, typename WT, int KM>
__global__ __launch_bounds__(256) void unpermute_dx_kernel(
    const ET* __restrict__ dxp, const int32_t* __restrict__ assign_row,
    const int32_t* __restrict__ off, const float* __restrict__ dlogits, const WT* __restrict__ wg,
    int64_t T, int d, int k, int E, int S, int64_t rows_max, ET* __restrict__ dx,
    const float* __restrict__ xr) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int64_t rj[KM];
  bool live[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int r = assign_row[t * k + min(j, k - 1)];
    live[j] = j < k && r >= 0 && r < rows_max;
    rj[j] = r;
  }
  const int64_t rs = S ? (int64_t)clamp_off(off, E, rows_max) + t : rows_max;
  const bool shared = rs < rows_max;
  int64_t first = shared ? rs : -1;
#pragma unroll
  for (int j = KM - 1; j >= 0; --j)
    if (live[j]) first = rj[j];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (!live[j]) rj[j] = first;
  const float* dl = dlogits + t * E;
  for (int c = lane * 8; c < d; c += 512) {
    // the expert-row loads (from HBM) issued first, the router term's weight
    // rows (cached) after them
    float a[KM][8], as[8];
    if (first >= 0) {
#pragma unroll
      for (int j = 0; j < KM; ++j) load8(dxp + rj[j] * d + c, a[j]);
      load8(dxp + (shared ? rs : first) * d + c, as);
    }
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (xr) load8(xr + t * d + c, v);
    for (int e0 = 0; e0 < (xr ? 0 : E); e0 += 8) {
      float wv[8][8], g[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = min(e0 + u, E - 1);
        load8(wg + (int64_t)e * d + c, wv[u]);
        g[u] = dl[e];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = e0 + u < E ? fmaf(g[u], wv[u][q], v[q]) : v[q];
    }
    if (first >= 0) {
#pragma unroll
      for (int j = 0; j < KM; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = live[j] ? v[q] + a[j][q] : v[q];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = shared ? v[q] + as[q] : v[q];
    }
    store8(dx + t * d + c, v);
  }
}

template <typename ET, typename WT>
static void launch_unpermute_dx(dim3 grid, hipStream_t s, const ET* dxp, const int32_t* assign_row,
                                const int32_t* off, const float* dlogits, const WT* wg, int64_t T,
                                int d, int k, int E, int S, int64_t rows_max, ET* dx,
                                const float* xr) {
  if (k <= 2)
    hipLaunchKernelGGL((unpermute_dx_kernel<ET, WT, 2>), grid, dim3(256), 0, s, dxp, assign_row,
                       off, dlogits, wg, T, d, k, E, S, rows_max, dx, xr);
  else if (k <= 4)
    hipLaunchKernelGGL((unpermute_dx_kernel<ET, WT, 4>), grid, dim3(256), 0, s, dxp, assign_row,
                       off, dlogits, wg, T, d, k, E, S, rows_max, dx, xr);
  else
    hipLaunchKernelGGL((unpermute_dx_kernel<ET, WT, MOE_MAX_TOP_K>), grid, dim3(256), 0, s, dxp,
                       assign_row, off, dlogits, wg, T, d, k, E, S, rows_max, dx, xr);
}

template <typename ET>
static void combine_bwd_t(const moe_config& c, const void* dy, const void* y_perm,
                          const moe_routing& r, void* dyp, float* dgate, hipStream_t s) {
  const int64_t T = c.tokens;
  hipLaunchKernelGGL(combine_bwd_kernel<ET>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
                     (const ET*)dy, (const ET*)y_perm, r.topk_gate, r.assign_row, r.expert_offsets,
                     T, (int)c.d_model, c.top_k, c.num_experts, c.num_shared_experts, rows_max(c),
                     (ET*)dyp, dgate);
}

hipError_t launch_combine_backward(const moe_config& c, const void* dy, const void* y_perm,
                                   const moe_routing& r, void* dyp, float* dgate, hipStream_t s) {
  if (c.act_dtype == MOE_BF16)
    combine_bwd_t<bf16>(c, dy, y_perm, r, dyp, dgate, s);
  else
    combine_bwd_t<float>(c, dy, y_perm, r, dyp, dgate, s);
  return hipGetLastError();
}

hipError_t launch_router_backward(const moe_config& c, const moe_routing& r, const moe_stats* stats,
                                  const float* dgate, float aux_coef, float z_coef, float* dlogits,
                                  hipStream_t s) {
  const int64_t T = c.tokens;
  const int E = c.num_experts;
  const int64_t per_block = 256 / (E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64)));   // tokens
  hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)((T + per_block - 1) / per_block)), dim3(256), 0, s, r.logits,
                     r.topk_idx, dgate, stats->counts_pre, T, c.num_experts, c.top_k,
                     (int)(c.score_fn == MOE_SCORE_SIGMOID), aux_coef, z_coef, dlogits);
  return hipGetLastError();
}

template <typename ET>
static void dx_t(const moe_config& c, const float* dlogits, const void* dxp, const moe_routing& r,
                 const moe_weights& w, const moe_grads& gr, hipStream_t s, const float* xr) {
  const int64_t T = c.tokens;
  const dim3 ug((unsigned)((T + 3) / 4));
  const int d = (int)c.d_model, k = c.top_k, E = c.num_experts, S = c.num_shared_experts;
  if (c.router_dtype == MOE_BF16)
    launch_unpermute_dx<ET, bf16>(ug, s, (const ET*)dxp, r.assign_row, r.expert_offsets, dlogits,
                                  (const bf16*)w.w_gate, T, d, k, E, S, rows_max(c), (ET*)gr.dx, xr);
  else
    launch_unpermute_dx<ET, float>(ug, s, (const ET*)dxp, r.assign_row, r.expert_offsets, dlogits,
                                   (const float*)w.w_gate, T, d, k, E, S, rows_max(c), (ET*)gr.dx, xr);
}

hipError_t launch_router_bias_and_dx(const moe_config& c, const float* dlogits, const void* dxp,
                                     const moe_routing& r, const moe_weights& w,
                                     const moe_grads& gr, hipStream_t s, const float* xr) {
  if (c.has_gate_bias)
    hipLaunchKernelGGL(gate_bias_grad_kernel, dim3(c.num_experts), dim3(256), 0, s, dlogits,
                       (int64_t)c.tokens, c.num_experts, gr.db_gate);
  if (c.act_dtype == MOE_BF16)
    dx_t<bf16>(c, dlogits, dxp, r, w, gr, s, xr);
  else
    dx_t<float>(c, dlogits, dxp, r, w, gr, s, xr);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers
hipError_t launch_act_rows(const moe_config& c, const void* z, const int32_t* off, void* h,
                           hipStream_t s) {
  if (c.act_dtype != MOE_BF16) return launch_act_rows_f32(c, z, off, h, s);
  const int G = c.num_experts + c.num_shared_experts;
  const int64_t n8 = rows_max(c) * c.d_ff / 8;
  const bf16* u = c.activation == MOE_ACT_SWIGLU ? (const bf16*)z + rows_max(c) * c.d_ff : nullptr;
  const int64_t blocks = (n8 + 255) / 256 < 4096 ? (n8 + 255) / 256 : 4096;
  hipLaunchKernelGGL(act_rows_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s,
                     (const bf16*)z, u, off, G, rows_max(c), (int)c.d_ff, c.activation, (bf16*)h);
  return hipGetLastError();
}

hipError_t launch_dswiglu(const moe_config& c, const void* dh, const void* z, void* dz,
                          const int32_t* off, hipStream_t s) {
  const int G = c.num_experts + c.num_shared_experts;
  const int64_t rmax = rows_max(c);
  const int64_t n8 = rmax * c.d_ff / 8;
  const int64_t blocks = (n8 + 255) / 256 < 4096 ? (n8 + 255) / 256 : 4096;
  hipLaunchKernelGGL(dswiglu_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s,
                     (const bf16*)dh, (const bf16*)z, (const bf16*)z + rmax * c.d_ff, off, G, rmax,
                     (int)c.d_ff, (bf16*)dz);
  return hipGetLastError();
}

hipError_t launch_backward_misc(const moe_config& c, const BwdLayout& B, const void* x,
                                const moe_weights& w, const moe_routing& r, const moe_stats* stats,
                                const moe_saved& sv, const void* dy, float aux_coef, float z_coef,
                                const moe_grads& gr, char* ws, hipStream_t s, int phase) {
  const int64_t T = c.tokens, rmax = rows_max(c);
  const int d = (int)c.d_model, F = (int)c.d_ff, E = c.num_experts, k = c.top_k;
  const int S = c.num_shared_experts, G = E + S;
  bf16* dyp = (bf16*)(ws + B.dyp);
  float* dgate = (float*)(ws + B.dgate);
  float* dlogits = (float*)(ws + B.dlogits);
  int32_t* po = (int32_t*)(ws + B.po);
  int32_t* so = po + (G + 1);
  if (phase == 0) {
    // combine and router backward, padded offsets
    hipError_t e = launch_combine_backward(c, dy, sv.y_perm, r, dyp, dgate, s);
    if (e != hipSuccess) return e;
    e = launch_router_backward(c, r, stats, dgate, aux_coef, z_coef, dlogits, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(64), 0, s, r.expert_offsets, G, rmax, po,
                       so);
    return hipGetLastError();
  }
  // phase 1 (after the dZ and dX GEMMs): weight gradients from the row buffers
  // (expert-sorted x rows gathered first), bias gradients, router weights, dx
  const unsigned kb = (unsigned)(B.ldk / 64);
  const bool sw = c.activation == MOE_ACT_SWIGLU;
  const int NZ = sw ? 2 : 1;   // dZ = [dz1 | du] for SwiGLU
  const bf16* dz = (const bf16*)(ws + B.dz);
  bf16* xp = (bf16*)(ws + B.xp);
  {
    const int64_t n = rmax * (d / 8);
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s,
                       (const bf16*)x, r.row_token, (const int32_t*)so, G, T, d, xp);
  }
  // dW2 = dYp^T H, dW1 = dz1^T Xp (dW3 = du^T Xp)
  hipError_t e = launch_wgrad(dyp, d, sv.h, F, so, G, E, d, F, rmax, gr.dw2, gr.dws2, s);
  if (e != hipSuccess) return e;
  e = launch_wgrad(dz, NZ * F, xp, d, so, G, E, F, d, rmax, gr.dw1, gr.dws1, s);
  if (e != hipSuccess) return e;
  if (sw) {
    e = launch_wgrad(dz + F, 2 * F, xp, d, so, G, E, F, d, rmax, gr.dw3, gr.dws3, s);
    if (e != hipSuccess) return e;
  }
  if (c.has_bias) {
    float* p2 = (float*)(ws + B.colsum2);
    float* p1 = (float*)(ws + B.colsum1);
    hipLaunchKernelGGL(colsum_rows_kernel, dim3(kb, (d + 511) / 512), dim3(256), 0, s,
                       (const bf16*)dyp, d, d, (const int32_t*)so, (const int32_t*)po, G, p2);
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3((d + 255) / 256, G), dim3(256), 0, s,
                       (const float*)p2, d, (const int32_t*)po, d, E, gr.db2, gr.dbs2);
    // b1 sits on W1 only: the dz1 columns (GELU / ReLU: tile sums from the dZ GEMM)
    if (sw) {
      hipLaunchKernelGGL(colsum_rows_kernel, dim3(kb, (F + 511) / 512), dim3(256), 0, s, dz, NZ * F,
                         F, (const int32_t*)so, (const int32_t*)po, G, p1);
      hipLaunchKernelGGL(colsum_reduce_kernel, dim3((F + 255) / 256, G), dim3(256), 0, s,
                         (const float*)p1, F, (const int32_t*)po, F, E, gr.db1, gr.dbs1);
    } else {
      hipLaunchKernelGGL(colsum_tiles_reduce_kernel, dim3((F + 255) / 256, G), dim3(256), 0, s,
                         (const float*)p1, r.expert_offsets, G, E, rmax, F,
                         (int)(B.ldk / 64), gr.db1, gr.dbs1);
    }
  }
  const int64_t n = (int64_t)E * d;
  if (B.gate_mfma) {
    // dlogits as two bf16 planes; dW_g = sum over token slices of the planes'
    // products with x (weight-gradient kernel, one group per slice, planes
    // [slice][hi, lo][E][d] added in that order); x's router term on MFMA
    bf16* dlp = (bf16*)(ws + B.dlp);
    int32_t* gso = (int32_t*)(ws + B.gso);
    const int64_t ne = T * E;
    hipLaunchKernelGGL(dlogit_planes_kernel, dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, s,
                       (const float*)dlogits, T, E, B.gate_slices, dlp, gso);
    e = launch_wgrad(dlp, 2 * E, x, d, gso, B.gate_slices, B.gate_slices, 2 * E, d, T,
                     (float*)(ws + B.gate_partial), nullptr, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gate_wgrad_reduce_kernel, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s,
                       (const float*)(ws + B.gate_partial), 2 * B.gate_slices, n, gr.dw_gate);
    e = launch_router_dx_gemm(c, dlp, w.w_gate, (float*)(ws + B.xr), s);
    if (e != hipSuccess) return e;
    return launch_router_bias_and_dx(c, dlogits, ws + B.dxp, r, w, gr, s,
                                     (const float*)(ws + B.xr));
  }
  hipLaunchKernelGGL(gate_wgrad_kernel, dim3((E + 7) / 8, (d + 511) / 512, B.gate_slices), dim3(256), 0, s,
                     (const bf16*)x, (const float*)dlogits, T, d, E, (int)B.gate_slice_len,
                     (float*)(ws + B.gate_partial));
  hipLaunchKernelGGL(gate_wgrad_reduce_kernel, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s,
                     (const float*)(ws + B.gate_partial), (int)B.gate_slices, n, gr.dw_gate);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_router_bias_and_dx(c, dlogits, ws + B.dxp, r, w, gr, s);
}

}  // namespace moe
