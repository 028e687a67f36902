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
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const bf16* __restrict__ dy, const bf16* __restrict__ y_perm, const float* __restrict__ gate,
    const int32_t* __restrict__ assign_row, const int32_t* __restrict__ off, int64_t T, int d, int k,
    int E, int S, int64_t rows_max, bf16* __restrict__ dyp, float* __restrict__ dgate) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const bf16* dyt = dy + t * d;
  for (int j = 0; j < k; ++j) {
    const int r = assign_row[t * k + j];
    float dot = 0.f;
    if (r >= 0 && r < rows_max) {
      const float g = gate[t * k + j];
      const bf16* yr = y_perm + (int64_t)r * d;
      bf16* out = dyp + (int64_t)r * d;
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
      bf16* out = dyp + r * d;
      for (int c = lane * 8; c < d; c += 512)
        *reinterpret_cast<uint4*>(out + c) = *reinterpret_cast<const uint4*>(dyt + c);
    }
  }
}

// ------------------------------------------------------------------ router backward
// One wavefront per token; lane l holds experts l, l + 64, l + 128, l + 192.
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
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
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
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float se = 0.f;
  float ex[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ex[i] = lane + 64 * i < E ? expf(hv[i] - m) : 0.f;
    se += ex[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) se += __shfl_xor(se, o, 64);
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
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dh[i] = p[i] * (ds[i] - dot);
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
    float dotq = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) dotq += dq[i] * (s[i] / tot);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dotq += __shfl_xor(dotq, o, 64);
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

// ------------------------------------------------------------------ transposes
// Batched bf16 transpose in[b][M][N] -> out[b][n][col0 + m] (out rows of ldo
// elements, so two matrices can be placed side by side) through a 64 x 64 LDS
// tile (16-byte loads and stores; M and N multiples of 64).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* __restrict__ in,
                                                             bf16* __restrict__ out, int M, int N,
                                                             int ldo, int col0) {
  __shared__ uint16_t tile[64][66];
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  const int64_t b = blockIdx.z;
  const bf16* src = in + b * (int64_t)M * N;
  bf16* dst = out + b * (int64_t)N * ldo + col0;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 3) + 32 * i, c = (tid & 7) * 8;
    const uint4 u = *reinterpret_cast<const uint4*>(src + (int64_t)(m0 + r) * N + n0 + c);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c + 2 * e] = (uint16_t)(w[e] & 0xffffu);
      tile[r][c + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 3) + 32 * i, c = (tid & 7) * 8;   // r: row of out (n), c: first m
    uint4 u;
    u.x = (uint32_t)tile[c + 0][r] | ((uint32_t)tile[c + 1][r] << 16);
    u.y = (uint32_t)tile[c + 2][r] | ((uint32_t)tile[c + 3][r] << 16);
    u.z = (uint32_t)tile[c + 4][r] | ((uint32_t)tile[c + 5][r] << 16);
    u.w = (uint32_t)tile[c + 6][r] | ((uint32_t)tile[c + 7][r] << 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)(n0 + r) * ldo + m0 + c) = u;
  }
}

// so[g]: expert_offsets clamped to [0, rows_max] and made non-decreasing, so the
// groups' rows never sum past rows_max; po[g] = sum over g' < g of the padded
// row count of group g' (its rows rounded up to a multiple of 128, at least
// 128), hence po[G] <= rows_max + 128 G (one thread; G <= 257).
__global__ void pad_offsets_kernel(const int32_t* __restrict__ off, int G, int64_t rows_max,
                                   int32_t* __restrict__ po, int32_t* __restrict__ so) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int acc = 0, prev = clamp_off(off, 0, rows_max);
  po[0] = 0;
  so[0] = prev;
  for (int g = 0; g < G; ++g) {
    int hi = clamp_off(off, g + 1, rows_max);
    hi = hi < prev ? prev : hi;
    const int r = hi - prev;
    const int p = r <= 128 ? 128 : (r + 127) & ~127;
    acc += p;
    po[g + 1] = acc;
    so[g + 1] = hi;
    prev = hi;
  }
}

// Expert-sorted rows -> transposed, group-padded layout for the weight
// gradient: out[c][k] for k in group g's padded range [po[g], po[g+1]) holds
// row r = so[g] + (k - po[g]) of the source (zero past the group's rows; so
// and po as written by pad_offsets_kernel).
// MODE 0: rows of src [rows][C]; MODE 1: token rows of src (x [T][C]) through
// row_token; MODE 2: act(src) (src = z, the saved pre-activation); MODE 3:
// silu(src) src2 (SwiGLU, src = z1, src2 = u). With
// partial != nullptr also writes the 64-row column sums of the (bf16) values
// of its block to partial[k / 64][c] (bias gradients).
template <int MODE>
__global__ __launch_bounds__(256) void transpose_rows_kernel(
    const bf16* __restrict__ src, const bf16* __restrict__ src2, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ so, const int32_t* __restrict__ po, int G, int64_t src_rows, int C,
    int ldk, int act, bf16* __restrict__ out, float* __restrict__ partial) {
  __shared__ float tile[64][65];
  const int k0 = blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  if (k0 >= po[G]) return;
  int lo = 0, hi = G;   // group of column k0: po[lo] <= k0 < po[lo + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (po[mid] <= k0) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int gs = so[g];
  const int R = so[g + 1] - gs;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kk = (tid >> 3) + 32 * i, c = (tid & 7) * 8;
    const int local = k0 + kk - po[g];
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (local < R) {
      int64_t row = gs + local;
      if (MODE == 1) {
        row = row_token[row];
        row = row < 0 ? 0 : (row >= src_rows ? src_rows - 1 : row);
      }
      load8(src + row * C + c0 + c, v);
      if (MODE == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32(f32_to_bf16_bits(act_bf16(act, v[e])));
      }
      if (MODE == 3) {
        float w[8];
        load8(src2 + row * C + c0 + c, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32(f32_to_bf16_bits(swiglu_h(v[e], w[e])));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[kk][c + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 3) + 32 * i, kc = (tid & 7) * 8;   // r: column of src, kc: first k
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[kc + e][r];
    store8(out + (int64_t)(c0 + r) * ldk + k0 + kc, v);
  }
  if (partial && tid < 64) {
    float sum = 0.f;
    for (int kk = 0; kk < 64; ++kk) sum += tile[kk][tid];
    partial[(int64_t)blockIdx.x * C + c0 + tid] = sum;
  }
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
// dW_g[e][c] = sum_t dlogits[t][e] x[t][c]. Block (8 experts, 1024 columns, a
// token slice): thread = 8 consecutive columns (one 16-byte load per token) x 8
// experts, the two halves of the block take alternate tokens and are added in
// LDS; the block's sums go to partial[slice][e][c] and
// gate_wgrad_reduce_kernel adds the slices in order.
__global__ __launch_bounds__(256) void gate_wgrad_kernel(const bf16* __restrict__ x,
                                                         const float* __restrict__ dlogits,
                                                         int64_t T, int d, int E, int slice_len,
                                                         float* __restrict__ partial) {
  __shared__ float red[128][65];
  const int e0 = blockIdx.x * 8;
  const int half = threadIdx.x >> 7;
  const int c = (blockIdx.y * 128 + (threadIdx.x & 127)) * 8;
  const int64_t t0 = (int64_t)blockIdx.z * slice_len;
  const int64_t t1 = t0 + slice_len < T ? t0 + slice_len : T;
  float acc[8][8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[e][u] = 0.f;
  if (c < d) {
    // four tokens per iteration, their loads issued together
    for (int64_t tb = t0 + half; tb < t1; tb += 8) {
      float xv[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t t = tb + 2 * q;
        if (t < t1) {
          load8(x + t * d + c, xv[q]);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) xv[q][u] = 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t t = tb + 2 * q;
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
  if (half == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int u = 0; u < 8; ++u) red[threadIdx.x & 127][e * 8 + u] = acc[e][u];
  }
  __syncthreads();
  if (half == 0 && c < d) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e0 + e < E) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = acc[e][u] + red[threadIdx.x][e * 8 + u];
        store8(partial + ((int64_t)blockIdx.z * E + e0 + e) * d + c, v);
      }
    }
  }
}

__global__ __launch_bounds__(256) void gate_wgrad_reduce_kernel(const float* __restrict__ partial,
                                                                int slices, int64_t n,
                                                                float* __restrict__ dw) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  int z = 0;
  for (; z + 8 <= slices; z += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[(z + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; z < slices; ++z) s += partial[z * n + i];
  dw[i] = s;
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

// ------------------------------------------------------------------ dx
// dx[t] = sum_j dXp[assign_row[t, j]] (kept choices, j order) + dXp[off[E] + t]
// (shared expert) + sum_e dlogits[t][e] W_g[e] (router), float32 sums, one
// rounding. One wavefront per token; lanes take 16-byte column chunks.
// KM >= k bounds the row slots at compile time. Loads are unconditional so a
// lane's loads issue before the first use (a load under a branch gets a wait
// of its own): W_g rows in batches of 8 (rows past E reread row E - 1), and
// row slots that are dropped or past k reread the token's first live row; all
// of them are masked out of the sums, which keep the order above.
template <typename WT, int KM>
__global__ __launch_bounds__(256) void unpermute_dx_kernel(
    const bf16* __restrict__ dxp, const int32_t* __restrict__ assign_row,
    const int32_t* __restrict__ off, const float* __restrict__ dlogits, const WT* __restrict__ wg,
    int64_t T, int d, int k, int E, int S, int64_t rows_max, bf16* __restrict__ dx) {
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
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int e0 = 0; e0 < E; e0 += 8) {
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
      float a[KM][8], as[8];
#pragma unroll
      for (int j = 0; j < KM; ++j) load8(dxp + rj[j] * d + c, a[j]);
      load8(dxp + (shared ? rs : first) * d + c, as);
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

template <typename WT>
static void launch_unpermute_dx(dim3 grid, hipStream_t s, const bf16* dxp, const int32_t* assign_row,
                                const int32_t* off, const float* dlogits, const WT* wg, int64_t T,
                                int d, int k, int E, int S, int64_t rows_max, bf16* dx) {
  if (k <= 2)
    hipLaunchKernelGGL((unpermute_dx_kernel<WT, 2>), grid, dim3(256), 0, s, dxp, assign_row, off,
                       dlogits, wg, T, d, k, E, S, rows_max, dx);
  else if (k <= 4)
    hipLaunchKernelGGL((unpermute_dx_kernel<WT, 4>), grid, dim3(256), 0, s, dxp, assign_row, off,
                       dlogits, wg, T, d, k, E, S, rows_max, dx);
  else
    hipLaunchKernelGGL((unpermute_dx_kernel<WT, MOE_MAX_TOP_K>), grid, dim3(256), 0, s, dxp,
                       assign_row, off, dlogits, wg, T, d, k, E, S, rows_max, dx);
}

// ------------------------------------------------------------------ launchers
hipError_t launch_act_rows(const moe_config& c, const void* z, const int32_t* off, void* h,
                           hipStream_t s) {
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
  const unsigned tb = (unsigned)((T + 3) / 4);
  if (phase == 0) {
    // combine and router backward, weight transposes
    hipLaunchKernelGGL(combine_bwd_kernel, dim3(tb), dim3(256), 0, s, (const bf16*)dy,
                       (const bf16*)sv.y_perm, r.topk_gate, r.assign_row, r.expert_offsets, T, d, k,
                       E, S, rmax, dyp, dgate);
    hipLaunchKernelGGL(router_bwd_kernel, dim3(tb), dim3(256), 0, s, r.logits, r.topk_idx, dgate,
                       stats->counts_pre, T, E, k, (int)(c.score_fn == MOE_SCORE_SIGMOID), aux_coef,
                       z_coef, dlogits);
    // W2^T [E][F][d]; W1^T [E][d][F], for SwiGLU [W1^T | W3^T] as [E][d][2F]
    const int NZ = c.activation == MOE_ACT_SWIGLU ? 2 : 1;
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3(F / 64, d / 64, E), dim3(256), 0, s,
                       (const bf16*)w.w2, (bf16*)(ws + B.w2t), d, F, d, 0);
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3(d / 64, F / 64, E), dim3(256), 0, s,
                       (const bf16*)w.w1, (bf16*)(ws + B.w1t), F, d, NZ * F, 0);
    if (NZ == 2)
      hipLaunchKernelGGL(transpose_bf16_kernel, dim3(d / 64, F / 64, E), dim3(256), 0, s,
                         (const bf16*)w.w3, (bf16*)(ws + B.w1t), F, d, 2 * F, F);
    if (S) {
      hipLaunchKernelGGL(transpose_bf16_kernel, dim3(F / 64, d / 64, 1), dim3(256), 0, s,
                         (const bf16*)w.ws2, (bf16*)(ws + B.ws2t), d, F, d, 0);
      hipLaunchKernelGGL(transpose_bf16_kernel, dim3(d / 64, F / 64, 1), dim3(256), 0, s,
                         (const bf16*)w.ws1, (bf16*)(ws + B.ws1t), F, d, NZ * F, 0);
      if (NZ == 2)
        hipLaunchKernelGGL(transpose_bf16_kernel, dim3(d / 64, F / 64, 1), dim3(256), 0, s,
                           (const bf16*)w.ws3, (bf16*)(ws + B.ws1t), F, d, 2 * F, F);
    }
    hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(64), 0, s, r.expert_offsets, G, rmax, po,
                       so);
    return hipGetLastError();
  }
  // phase 1 (after the dZ and dX GEMMs): transposed row buffers, weight
  // gradients, bias gradients, router weights, dx
  const int ldk = (int)B.ldk;
  const unsigned kb = (unsigned)(B.ldk / 64);
  const bool bias = c.has_bias;
  float* p2 = bias ? (float*)(ws + B.colsum2) : nullptr;
  float* p1 = bias ? (float*)(ws + B.colsum1) : nullptr;
  const bool sw = c.activation == MOE_ACT_SWIGLU;
  const int NZ = sw ? 2 : 1;   // dZ = [dz1 | du] for SwiGLU
  const bf16* z1 = (const bf16*)sv.z;
  const bf16* u = sw ? z1 + rmax * F : nullptr;
  hipLaunchKernelGGL((transpose_rows_kernel<0>), dim3(kb, d / 64), dim3(256), 0, s,
                     (const bf16*)dyp, (const bf16*)nullptr, (const int32_t*)nullptr,
                     (const int32_t*)so, po, G, rmax, d, ldk, c.activation, (bf16*)(ws + B.dypT),
                     p2);
  if (sw)
    hipLaunchKernelGGL((transpose_rows_kernel<3>), dim3(kb, F / 64), dim3(256), 0, s, z1, u,
                       (const int32_t*)nullptr, (const int32_t*)so, po, G, rmax, F, ldk,
                       c.activation, (bf16*)(ws + B.hT), (float*)nullptr);
  else
    hipLaunchKernelGGL((transpose_rows_kernel<2>), dim3(kb, F / 64), dim3(256), 0, s, z1,
                       (const bf16*)nullptr, (const int32_t*)nullptr, (const int32_t*)so, po, G, rmax,
                       F, ldk, c.activation, (bf16*)(ws + B.hT), (float*)nullptr);
  hipLaunchKernelGGL((transpose_rows_kernel<0>), dim3(kb, NZ * F / 64), dim3(256), 0, s,
                     (const bf16*)(ws + B.dz), (const bf16*)nullptr, (const int32_t*)nullptr,
                     (const int32_t*)so, po, G, rmax, NZ * F, ldk, c.activation,
                     (bf16*)(ws + B.dzT), p1);
  hipLaunchKernelGGL((transpose_rows_kernel<1>), dim3(kb, d / 64), dim3(256), 0, s, (const bf16*)x,
                     (const bf16*)nullptr, r.row_token, (const int32_t*)so, po, G, T, d, ldk,
                     c.activation, (bf16*)(ws + B.xT), (float*)nullptr);
  hipError_t e = launch_wgrad(ws + B.dypT, ws + B.hT, po, G, E, d, F, ldk, gr.dw2, gr.dws2, s);
  if (e != hipSuccess) return e;
  e = launch_wgrad(ws + B.dzT, ws + B.xT, po, G, E, F, d, ldk, gr.dw1, gr.dws1, s);
  if (e != hipSuccess) return e;
  if (sw) {
    // dW3 from the du rows of dZ^T
    e = launch_wgrad(ws + B.dzT + (size_t)F * ldk * 2, ws + B.xT, po, G, E, F, d, ldk, gr.dw3,
                     gr.dws3, s);
    if (e != hipSuccess) return e;
  }
  if (bias) {
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3((d + 255) / 256, G), dim3(256), 0, s,
                       (const float*)p2, d, (const int32_t*)po, d, E, gr.db2, gr.dbs2);
    // b1 sits on W1 only: the dz1 columns
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3((F + 255) / 256, G), dim3(256), 0, s,
                       (const float*)p1, NZ * F, (const int32_t*)po, F, E, gr.db1, gr.dbs1);
  }
  hipLaunchKernelGGL(gate_wgrad_kernel, dim3((E + 7) / 8, (d + 1023) / 1024, B.gate_slices), dim3(256), 0, s,
                     (const bf16*)x, (const float*)dlogits, T, d, E, (int)B.gate_slice_len,
                     (float*)(ws + B.gate_partial));
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL(gate_wgrad_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const float*)(ws + B.gate_partial), (int)B.gate_slices, n, gr.dw_gate);
  if (c.has_gate_bias)
    hipLaunchKernelGGL(gate_bias_grad_kernel, dim3(E), dim3(256), 0, s, (const float*)dlogits, T, E,
                       gr.db_gate);
  const dim3 ug((unsigned)((T + 3) / 4));
  if (c.router_dtype == MOE_BF16)
    launch_unpermute_dx<bf16>(ug, s, (const bf16*)(ws + B.dxp), r.assign_row, r.expert_offsets,
                              (const float*)dlogits, (const bf16*)w.w_gate, T, d, k, E, S, rmax,
                              (bf16*)gr.dx);
  else
    launch_unpermute_dx<float>(ug, s, (const bf16*)(ws + B.dxp), r.assign_row, r.expert_offsets,
                               (const float*)dlogits, (const float*)w.w_gate, T, d, k, E, S, rmax,
                               (bf16*)gr.dx);
  return hipGetLastError();
}

}  // namespace moe
