// The training path of float32 layers: the activation pass of the training
// forward and the whole backward, in float32 throughout. Every kernel computes
// one output element (or one 8-element run) per thread with plain FMA loops in
// a fixed order, so the results are deterministic; the float32 layers are the
// small ones (the page's basic layer), and their GEMMs are not worth MFMA
// tiling.
//
// Chain rule of the layer (MoE Training: Mixture of Experts, "Basic MoE
// Architecture" for the expert FFN, "3. Load Balancing" for L_aux; MoE From
// Scratch to DeepSeek V3 for the gated sum, the z-loss and the sigmoid router):
//   dYp[r] = g dy[t] for the kept row r of (t, j), dy[t] for the shared row;
//   dH = dYp W2_g;  dZ = dH act'(Z) (SwiGLU: dz1 = dH u silu'(z1), du = dH silu(z1));
//   dXp = dZ W1_g (+ du W3_g);  dx[t] = sum of its rows' dXp + dlogits[t] W_g;
//   dW2_g = dYp^T H,  dW1_g = dZ^T X,  dW3_g = du^T X,  db2_g = sum dYp,  db1_g = sum dZ;
//   dW_g = dlogits^T x,  db_g = sum_t dlogits.
// The combine and router steps share their kernels with the bf16 path.
#include <cstring>

#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ float act_f32(int act, float z) {
  return act == MOE_ACT_RELU ? fmaxf(z, 0.f) : gelu_erf(z);
}

// d/dz GELU(z) = Phi(z) + z phi(z) (exact erf form); ReLU' = 1 for z > 0.
__device__ __forceinline__ float dact_f32(int act, float z) {
  if (act == MOE_ACT_RELU) return z > 0.f ? 1.0f : 0.0f;
  const float Phi = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
  const float phi = 0.3989422804014327f * expf(-0.5f * z * z);
  return fmaf(z, phi, Phi);
}

__device__ __forceinline__ int64_t clamped(const int32_t* __restrict__ off, int g, int64_t rmax) {
  const int64_t v = off[g];
  return v < 0 ? 0 : (v > rmax ? rmax : v);
}

// Group of row r: the g with off[g] <= r < off[g + 1] (offsets clamped to
// [0, rmax]), or -1 when r is past the last group's rows.
__device__ __forceinline__ int group_of(const int32_t* __restrict__ off, int G, int64_t rmax,
                                        int64_t r) {
  if (r >= clamped(off, G, rmax)) return -1;
  int lo = 0, hi = G - 1;   // the last g with off[g] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (clamped(off, mid, rmax) <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

}  // namespace

// h[r][f] = act(z[r][f]) (SwiGLU: silu(z1) u) for the rows of the groups.
__global__ __launch_bounds__(256) void act_rows_f32_kernel(const float* __restrict__ z,
                                                           const float* __restrict__ u,
                                                           const int32_t* __restrict__ off, int G,
                                                           int64_t rmax, int F, int act,
                                                           float* __restrict__ h) {
  const int64_t n = clamped(off, G, rmax) * F;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    h[i] = u ? silu(z[i]) * u[i] : act_f32(act, z[i]);
}

// Grouped product with the weight read as stored, C[r][n] = sum_k A[r][k]
// W_g[k][n] (+ sum_k A2[r][k] W2_g[k][n]), W_g = W + g K N for g < E, Ws for the
// shared group; then C *= act'(Z[r][n]) when Z is given. Rows of A (and A2)
// are lda floats apart; C and Z rows are N floats apart. One thread per (r, n):
// blockIdx.x = row, blockIdx.y = 256 columns.
__global__ __launch_bounds__(256) void gemm_nn_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ A2, int64_t lda,
    const float* __restrict__ W, const float* __restrict__ Ws, const float* __restrict__ W2,
    const float* __restrict__ Ws2, int E, int G, const int32_t* __restrict__ off, int64_t rmax,
    int K, int N, const float* __restrict__ Z, int act, float* __restrict__ C) {
  const int64_t r = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  const int g = group_of(off, G, rmax, r);
  if (g < 0 || n >= N) return;
  const float* w = g < E ? W + (int64_t)g * K * N : Ws;
  const float* a = A + r * lda;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(a[k], w[(int64_t)k * N + n], s);
  if (A2) {
    const float* w2 = g < E ? W2 + (int64_t)g * K * N : Ws2;
    const float* a2 = A2 + r * lda;
    for (int k = 0; k < K; ++k) s = fmaf(a2[k], w2[(int64_t)k * N + n], s);
  }
  if (Z) s *= dact_f32(act, Z[r * N + n]);
  C[r * N + n] = s;
}

// SwiGLU, elementwise: dz1 = dH u silu'(z1), du = dH silu(z1), written as
// row r of dZ [rows][2F] (dz1 in columns 0..F-1, du in F..2F-1).
__global__ __launch_bounds__(256) void dswiglu_f32_kernel(const float* __restrict__ dh,
                                                          const float* __restrict__ z1,
                                                          const float* __restrict__ u,
                                                          const int32_t* __restrict__ off, int G,
                                                          int64_t rmax, int F,
                                                          float* __restrict__ dz) {
  const int64_t n = clamped(off, G, rmax) * F;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / F, c = i - r * F;
    const float a = z1[i], sg = 1.0f / (1.0f + expf(-a));
    dz[r * 2 * F + c] = dh[i] * u[i] * sg * (1.0f + a * (1.0f - sg));
    dz[r * 2 * F + F + c] = dh[i] * a * sg;
  }
}

// Per group, out_g[i][j] = sum over the group's rows r (ascending) of
// A[r][i] B[b(r)][j], with b(r) = brows[r] when brows is given, else r; with
// B == nullptr, out_g[i] = sum_r A[r][i] (bias gradients). Rows of A are lda
// floats apart, rows of B ldb. Group g < E writes out + g NA NB (or + g NA),
// the shared group writes out_s. With off == nullptr there is one group of
// rows [0, rmax) writing out. One thread per output: blockIdx.x = (g, i),
// blockIdx.y = 256 values of j.
__global__ __launch_bounds__(256) void wgrad_f32_kernel(
    const float* __restrict__ A, int64_t lda, const float* __restrict__ B, int64_t ldb,
    const int32_t* __restrict__ brows, const int32_t* __restrict__ off, int E, int G, int64_t rmax,
    int NA, int NB, float* __restrict__ out, float* __restrict__ out_s) {
  const int g = blockIdx.x / NA, i = blockIdx.x - g * NA;
  const int j = blockIdx.y * 256 + threadIdx.x;
  const int nb = B ? NB : 1;
  if (j >= nb) return;
  int64_t r0 = 0, r1 = rmax;
  if (off) {
    r0 = clamped(off, g, rmax);
    r1 = clamped(off, g + 1, rmax);
    if (r1 < r0) r1 = r0;
  }
  float s = 0.f;
  for (int64_t r = r0; r < r1; ++r) {
    const float a = A[r * lda + i];
    s = B ? fmaf(a, B[(int64_t)(brows ? brows[r] : r) * ldb + j], s) : s + a;
  }
  float* o = (off && g >= E) ? out_s : out + (int64_t)g * NA * nb;
  if (o) o[(int64_t)i * nb + j] = s;
}

hipError_t launch_act_rows_f32(const moe_config& c, const void* z, const int32_t* off, void* h,
                               hipStream_t s) {
  const int G = c.num_experts + c.num_shared_experts;
  const int64_t rmax = rows_max(c), F = c.d_ff;
  const float* u = c.activation == MOE_ACT_SWIGLU ? (const float*)z + rmax * F : nullptr;
  const int64_t blocks = (rmax * F + 255) / 256 < 4096 ? (rmax * F + 255) / 256 : 4096;
  hipLaunchKernelGGL(act_rows_f32_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0,
                     s, (const float*)z, u, off, G, rmax, (int)F, c.activation, (float*)h);
  return hipGetLastError();
}

BwdLayout backward_layout_f32(const moe_config& c) {
  BwdLayout B;
  memset(&B, 0, sizeof(B));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const int64_t T = c.tokens, d = c.d_model, F = c.d_ff, rmax = rows_max(c);
  const int64_t NZ = c.activation == MOE_ACT_SWIGLU ? 2 : 1;
  B.dyp = take((size_t)(rmax * d * 4));
  B.dgate = take((size_t)(T * c.top_k * 4));
  B.dlogits = take((size_t)(T * c.num_experts * 4));
  B.dz = take((size_t)(rmax * NZ * F * 4));
  B.dh = take(NZ == 2 ? (size_t)(rmax * F * 4) : 0);
  B.dxp = take((size_t)(rmax * d * 4));
  B.total = off;
  return B;
}

hipError_t launch_backward_f32(const moe_config& c, const BwdLayout& B, const void* x,
                               const moe_weights& w, const moe_routing& r, const moe_stats* stats,
                               const moe_saved& sv, const void* dy, float aux_coef, float z_coef,
                               const moe_grads& gr, char* ws, hipStream_t s) {
  const int64_t T = c.tokens, rmax = rows_max(c);
  const int d = (int)c.d_model, F = (int)c.d_ff, E = c.num_experts, k = c.top_k;
  const int S = c.num_shared_experts, G = E + S;
  const bool sw = c.activation == MOE_ACT_SWIGLU;
  const int NZ = sw ? 2 : 1;
  float* dyp = (float*)(ws + B.dyp);
  float* dgate = (float*)(ws + B.dgate);
  float* dlogits = (float*)(ws + B.dlogits);
  float* dz = (float*)(ws + B.dz);
  const float* h = (const float*)sv.h;   // act(z) as the training forward kept it
  float* dxp = (float*)(ws + B.dxp);
  const float* z1 = (const float*)sv.z;
  const float* u = sw ? z1 + rmax * F : nullptr;
  const int32_t* off = r.expert_offsets;
  hipError_t e = launch_combine_backward(c, dy, sv.y_perm, r, dyp, dgate, s);
  if (e != hipSuccess) return e;
  e = launch_router_backward(c, r, stats, dgate, aux_coef, z_coef, dlogits, s);
  if (e != hipSuccess) return e;
  const unsigned rows = (unsigned)(rmax > 0 ? rmax : 1);
  // dZ (GELU, ReLU: the activation derivative applied in the product's epilogue)
  float* dhz = sw ? (float*)(ws + B.dh) : dz;
  hipLaunchKernelGGL(gemm_nn_f32_kernel, dim3(rows, (F + 255) / 256), dim3(256), 0, s,
                     (const float*)dyp, (const float*)nullptr, (int64_t)d, (const float*)w.w2,
                     (const float*)w.ws2, (const float*)nullptr, (const float*)nullptr, E, G, off,
                     rmax, d, F, sw ? (const float*)nullptr : z1, c.activation, dhz);
  if (sw) {
    const int64_t blocks = (rmax * F + 255) / 256 < 4096 ? (rmax * F + 255) / 256 : 4096;
    hipLaunchKernelGGL(dswiglu_f32_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0,
                       s, (const float*)dhz, z1, u, off, G, rmax, F, dz);
  }
  // dXp = dz1 W1 (+ du W3)
  hipLaunchKernelGGL(gemm_nn_f32_kernel, dim3(rows, (d + 255) / 256), dim3(256), 0, s,
                     (const float*)dz, sw ? (const float*)dz + F : (const float*)nullptr,
                     (int64_t)NZ * F, (const float*)w.w1, (const float*)w.ws1,
                     (const float*)w.w3, (const float*)w.ws3, E, G, off, rmax, F, d,
                     (const float*)nullptr, c.activation, dxp);
  // weight and bias gradients of the experts
  hipLaunchKernelGGL(wgrad_f32_kernel, dim3(G * d, (F + 255) / 256), dim3(256), 0, s,
                     (const float*)dyp, (int64_t)d, (const float*)h, (int64_t)F,
                     (const int32_t*)nullptr, off, E, G, rmax, d, F, gr.dw2, gr.dws2);
  hipLaunchKernelGGL(wgrad_f32_kernel, dim3(G * F, (d + 255) / 256), dim3(256), 0, s,
                     (const float*)dz, (int64_t)NZ * F, (const float*)x, (int64_t)d, r.row_token,
                     off, E, G, rmax, F, d, gr.dw1, gr.dws1);
  if (sw)
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3(G * F, (d + 255) / 256), dim3(256), 0, s,
                       (const float*)dz + F, (int64_t)NZ * F, (const float*)x, (int64_t)d,
                       r.row_token, off, E, G, rmax, F, d, gr.dw3, gr.dws3);
  if (c.has_bias) {
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3(G * d, 1), dim3(256), 0, s, (const float*)dyp,
                       (int64_t)d, (const float*)nullptr, (int64_t)0, (const int32_t*)nullptr, off,
                       E, G, rmax, d, 0, gr.db2, gr.dbs2);
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3(G * F, 1), dim3(256), 0, s, (const float*)dz,
                       (int64_t)NZ * F, (const float*)nullptr, (int64_t)0,
                       (const int32_t*)nullptr, off, E, G, rmax, F, 0, gr.db1, gr.dbs1);
  }
  // router weights: dW_g = dlogits^T x over the T tokens (one group)
  hipLaunchKernelGGL(wgrad_f32_kernel, dim3(E, (d + 255) / 256), dim3(256), 0, s,
                     (const float*)dlogits, (int64_t)E, (const float*)x, (int64_t)d,
                     (const int32_t*)nullptr, (const int32_t*)nullptr, E, 1, T, E, d, gr.dw_gate,
                     (float*)nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_router_bias_and_dx(c, dlogits, dxp, r, w, gr, s);
}

}  // namespace moe
