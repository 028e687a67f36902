// Capacity-limited dispatch: per-chunk histogram with a stable in-chunk rank,
// a scan over (chunk, expert) that applies the capacity, and the scatter of
// the routing maps together with the gather of token rows into the
// expert-sorted buffer.
//
// MoE From Scratch to DeepSeek V3, "Token Dropping" (a full expert buffer drops
// the extra tokens); MoE Training Guide, "Core MoE Parameters" items 4-7
// (capacity factor, minimum capacity, no-drop mode) and "Monitoring".
// Queue order: assignment (t, j) has priority a = j*T + t (k-major, then
// token-ascending); its position in its expert's queue is the number of
// earlier assignments to the same expert. Ranks come from ordered counting
// (wave ballots + per-wave counts), never from atomic return order, so every
// integer output is deterministic.
#include "moe_internal.h"

namespace moe {

// Per-expert exclusive scan over chunks (queue base of each chunk), counts
// before and after capacity, expert offsets, and the statistics that need the
// counts (f_i, L_aux with the router's P_i); one block of 256 threads.
__device__ __forceinline__ void dispatch_scan_block(
    const int32_t* __restrict__ chunk_hist, int32_t* __restrict__ chunk_base, int chunks, int E,
    int64_t T, int k, int S, int64_t cap, int32_t* __restrict__ expert_offsets,
    moe_stats* __restrict__ stats, int* sc, double* red) {
  const int e = threadIdx.x;
  int pre = 0;
  if (e < E) {
    // eight chunk counts loaded together per round, unconditionally (past the
    // last chunk: the last one again, not added), so their round trips overlap
    for (int c0 = 0; c0 < chunks; c0 += 8) {
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        h[u] = chunk_hist[(int64_t)min(c0 + u, chunks - 1) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u < chunks) {
          chunk_base[(int64_t)(c0 + u) * E + e] = pre;
          pre += h[u];
        }
      }
    }
  }
  const int kept = (e < E) ? (cap < 0 ? pre : (int)((int64_t)pre < cap ? pre : cap)) : 0;
  sc[e] = kept;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  const int R = sc[255];
  if (e < E) expert_offsets[e] = sc[e] - kept;
  if (e == 0) {
    expert_offsets[E] = R;
    if (S) expert_offsets[E + 1] = R + (int)T;
  }
  const int64_t A = T * k;
  stats->counts_pre[e] = pre;
  stats->counts_kept[e] = kept;
  const double f = (e < E) ? (double)pre / (double)A : 0.0;
  stats->frac[e] = (float)f;
  red[e] = (e < E) ? f * (double)stats->prob_mean[e] : 0.0;
  __syncthreads();
  if (e == 0) {
    double s = 0.0;
    for (int i = 0; i < E; ++i) s += red[i];
    stats->l_aux = (float)((double)E * s);
    stats->capacity = cap < 0 ? -1 : (int)(cap < 0x7fffffff ? cap : 0x7fffffff);
    stats->kept = R;
    stats->dropped = (int)(A - R);
    stats->reserved[0] = stats->reserved[1] = stats->reserved[2] = 0;
  }
}

// Blocks b < chunks: block b ranks kRankChunk consecutive assignments, 256 per
// round, and writes its chunk's per-expert counts. Blocks chunks .. chunks +
// E + 1 (route_blocks > 0): column b - chunks of the router statistics
// (route_stats_column over route_blocks partial rows), which the scan kernel
// after this launch reads for L_aux.
__global__ __launch_bounds__(256) void dispatch_rank_kernel(const int32_t* __restrict__ topk_idx,
                                                            int64_t T, int k, int E, int64_t A,
                                                            int32_t* __restrict__ local_rank,
                                                            int32_t* __restrict__ chunk_hist,
                                                            int chunks, const float* __restrict__ rp,
                                                            int route_blocks,
                                                            moe_stats* __restrict__ stats) {
  __shared__ int hist[MOE_MAX_EXPERTS];
  __shared__ int wcount[4][MOE_MAX_EXPERTS];
  __shared__ double red[256];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < chunks) {
  const int lane = tid & 63;
  const int w = tid >> 6;
  hist[tid] = 0;
  const int64_t a0 = (int64_t)blockIdx.x * kRankChunk;
  for (int r = 0; r < kRankChunk / 256; ++r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wcount[i][tid] = 0;
    __syncthreads();
    const int64_t a = a0 + r * 256 + tid;
    int e = 511;  // sentinel: no assignment / index out of range
    if (a < A) {
      const int64_t j = a / T;
      const int64_t t = a - j * T;
      const int v = topk_idx[t * k + j];
      if (v >= 0 && v < E) e = v;
    }
    // lanes holding the same expert id
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank_w = __popcll(peers & ((1ull << lane) - 1ull));
    if (e < E && rank_w == 0) wcount[w][e] = __popcll(peers);
    __syncthreads();
    if (e < E) {
      int rank = hist[e] + rank_w;
      for (int ww = 0; ww < w; ++ww) rank += wcount[ww][e];
      local_rank[a] = rank;
    }
    __syncthreads();
    hist[tid] += wcount[0][tid] + wcount[1][tid] + wcount[2][tid] + wcount[3][tid];
    __syncthreads();
  }
  if (tid < E) chunk_hist[(int64_t)blockIdx.x * E + tid] = hist[tid];
  } else {
    route_stats_column(rp, route_blocks, E, T, stats, (int)blockIdx.x - chunks, red);
  }
}

// Single block: the chunk scan, counts, offsets and statistics
// (dispatch_scan_block).
__global__ __launch_bounds__(256) void dispatch_scan_kernel(
    const int32_t* __restrict__ chunk_hist, int32_t* __restrict__ chunk_base, int chunks, int E,
    int64_t T, int k, int S, int64_t cap, int32_t* __restrict__ expert_offsets,
    moe_stats* __restrict__ stats) {
  __shared__ int sc[256];
  __shared__ double red[256];
  dispatch_scan_block(chunk_hist, chunk_base, chunks, E, T, k, S, cap, expert_offsets, stats, sc,
                      red);
}

// One wavefront per assignment (and per shared-expert row): writes the maps
// and copies the token row with 16-byte accesses.
template <typename ET>
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const ET* __restrict__ x, int64_t T, int k, int E, int S,
    int64_t cap, int d, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ assign_row, ET* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t A = T * k;
  const int64_t a = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int64_t t, row = -1;
  if (a < A) {
    const int64_t j = a / T;
    t = a - j * T;
    const int e = topk_idx[t * k + j];
    if (e >= 0 && e < E) {
      const int64_t pos = (int64_t)chunk_base[(a / kRankChunk) * E + e] + local_rank[a];
      if (cap < 0 || pos < cap) row = (int64_t)expert_offsets[e] + pos;
    }
    if (lane == 0) {
      assign_row[t * k + j] = (int32_t)row;
      if (row >= 0) row_token[row] = (int32_t)t;
    }
  } else if (S && a < A + T) {
    t = a - A;
    row = (int64_t)expert_offsets[E] + t;
    if (lane == 0) row_token[row] = (int32_t)t;
  } else {
    return;
  }
  if (row < 0 || x_perm == nullptr) return;
  const char* src = reinterpret_cast<const char*>(x + t * d);
  char* dst = reinterpret_cast<char*>(x_perm + row * d);
  const int64_t bytes = (int64_t)d * sizeof(ET);
  for (int64_t off = (int64_t)lane * 16; off < bytes; off += 64 * 16)
    *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(src + off);
}

// The maps alone (no row copy: the forward's GEMM 1 gathers the token rows
// itself): one thread per assignment (and per shared-expert row).
__global__ __launch_bounds__(256) void dispatch_maps_kernel(
    const int32_t* __restrict__ topk_idx, int64_t T, int k, int E, int S, int64_t cap,
    const int32_t* __restrict__ local_rank, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ expert_offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ assign_row) {
  const int64_t A = T * k;
  const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a < A) {
    const int64_t j = a / T;
    const int64_t t = a - j * T;
    const int e = topk_idx[t * k + j];
    int64_t row = -1;
    if (e >= 0 && e < E) {
      const int64_t pos = (int64_t)chunk_base[(a / kRankChunk) * E + e] + local_rank[a];
      if (cap < 0 || pos < cap) row = (int64_t)expert_offsets[e] + pos;
    }
    assign_row[t * k + j] = (int32_t)row;
    if (row >= 0) row_token[row] = (int32_t)t;
  } else if (S && a < A + T) {
    const int64_t t = a - A;
    row_token[(int64_t)expert_offsets[E] + t] = (int32_t)t;
  }
}

hipError_t launch_permute(const moe_config& c, const WsLayout& L, int64_t cap,
                          const int32_t* topk_idx, const void* x, int32_t* expert_offsets,
                          int32_t* row_token, int32_t* assign_row, void* x_perm, moe_stats* stats,
                          char* ws, hipStream_t s, int route_blocks) {
  const int64_t T = c.tokens;
  const int k = c.top_k, E = c.num_experts, S = c.num_shared_experts;
  const int64_t A = T * k;
  int32_t* local_rank = reinterpret_cast<int32_t*>(ws + L.local_rank);
  int32_t* chunk_hist = reinterpret_cast<int32_t*>(ws + L.chunk_hist);
  int32_t* chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  const int extra = route_blocks > 0 ? E + 2 : 0;
  hipLaunchKernelGGL(dispatch_rank_kernel, dim3((unsigned)(L.chunks + extra)), dim3(256), 0, s,
                     topk_idx, T, k, E, A, local_rank, chunk_hist, L.chunks,
                     reinterpret_cast<const float*>(ws + L.route_partials), route_blocks, stats);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(256), 0, s, chunk_hist, chunk_base,
                     L.chunks, E, T, k, S, cap, expert_offsets, stats);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t waves = A + S * T;
  if (!x_perm) {
    hipLaunchKernelGGL(dispatch_maps_kernel, dim3((unsigned)((waves + 255) / 256)), dim3(256), 0, s,
                       topk_idx, T, k, E, S, cap, local_rank, chunk_base, expert_offsets, row_token,
                       assign_row);
    return hipGetLastError();
  }
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  if (c.act_dtype == MOE_BF16)
    hipLaunchKernelGGL((dispatch_scatter_kernel<bf16>), dim3(blocks), dim3(256), 0, s, topk_idx,
                       (const bf16*)x, T, k, E, S, cap, (int)c.d_model, local_rank, chunk_base,
                       expert_offsets, row_token, assign_row, (bf16*)x_perm);
  else
    hipLaunchKernelGGL((dispatch_scatter_kernel<float>), dim3(blocks), dim3(256), 0, s, topk_idx,
                       (const float*)x, T, k, E, S, cap, (int)c.d_model, local_rank, chunk_base,
                       expert_offsets, row_token, assign_row, (float*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
