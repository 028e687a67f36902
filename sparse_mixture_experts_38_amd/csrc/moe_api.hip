// C ABI of the MoE-layer forward: validation, capacity, workspace layout and
// the entry points declared in moe.h. Host code only; kernels live in the
// other sources.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moe_internal.h"

namespace moe {

static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout workspace_layout(const moe_config& c) {
  WsLayout L;
  memset(&L, 0, sizeof(L));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const int64_t T = c.tokens;
  const int E = c.num_experts, k = c.top_k, S = c.num_shared_experts;
  const int64_t A = T * k;
  const int gpb = 256 / route_lanes(E);
  const int64_t groups = (T + gpb - 1) / gpb;
  const int64_t iters = groups > 1024 ? (groups + 1023) / 1024 : 1;
  L.route_iters = (int)iters;
  L.route_blocks = (int)(groups > 0 ? (groups + iters - 1) / iters : 1);
  L.logits = take((size_t)T * E * sizeof(float));
  // (the MFMA router for a few experts writes one row per 32 tokens instead)
  const int64_t pblocks = std::max<int64_t>(L.route_blocks, (T + 31) / 32);
  L.route_partials = take((size_t)pblocks * (E + 1) * sizeof(float));
  L.router_planes = take((size_t)router_kparts(c) * T * E * sizeof(float));
  L.end_route = off;
  L.chunks = (int)(A > 0 ? (A + kRankChunk - 1) / kRankChunk : 1);
  L.chunk_hist = take((size_t)L.chunks * E * sizeof(int32_t));
  L.chunk_base = take((size_t)L.chunks * E * sizeof(int32_t));
  L.local_rank = take((size_t)A * sizeof(int32_t));
  L.end_permute = off;
  L.rows_max = A + (int64_t)S * T;
  const size_t es = c.act_dtype == MOE_BF16 ? 2 : 4;
  L.h = take((size_t)L.rows_max * c.d_ff * es);
  L.rest_bytes = rest_partial_bytes(c, 0);
  L.rest_partial = take(L.rest_bytes);
  L.end_ffn = off;
  L.y_perm = take((size_t)L.rows_max * c.d_model * es);
  L.total = off;
  return L;
}

BwdLayout backward_layout(const moe_config& c) {
  BwdLayout B;
  memset(&B, 0, sizeof(B));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const int64_t T = c.tokens, d = c.d_model, F = c.d_ff;
  const int E = c.num_experts, k = c.top_k, S = c.num_shared_experts, G = E + S;
  const int64_t rmax = rows_max(c);
  B.ldk = (rmax + 128 * (int64_t)G + 127) / 128 * 128;
  B.dyp = take((size_t)(rmax * d * 2));
  B.dgate = take((size_t)(T * k * 4));
  B.dlogits = take((size_t)(T * E * 4));
  const int64_t NZ = c.activation == MOE_ACT_SWIGLU ? 2 : 1;   // SwiGLU: [dz1 | du]
  B.dz = take((size_t)(rmax * NZ * F * 2));
  B.dh = take(NZ == 2 ? (size_t)(rmax * F * 2) : 0);
  B.dxp = take((size_t)(rmax * d * 2));
  B.po = take((size_t)(G + 1) * 8);   // po [G + 1], then the sanitized offsets [G + 1]
  B.xp = take((size_t)(rmax * d * 2));
  B.colsum1 = take(c.has_bias ? (size_t)(B.ldk / 64 * F * 4) : 0);
  B.colsum2 = take(c.has_bias ? (size_t)(B.ldk / 64 * d * 4) : 0);
  // router weight gradient: about 256 blocks of (8 experts x 512 columns x a
  // token slice), slices of at least 64 tokens
  const int64_t xy = (int64_t)((E + 7) / 8) * ((d + 511) / 512);
  int64_t slices = 256 / xy;
  slices = slices < 1 ? 1 : (slices > 256 ? 256 : slices);
  if (slices > T / 64) slices = T / 64 > 0 ? T / 64 : 1;
  const int64_t slice_len = T > 0 ? (T + slices - 1) / slices : 1;
  B.gate_slice_len = (int)slice_len;
  B.gate_slices = (int)(T > 0 ? (T + slice_len - 1) / slice_len : 1);
  B.gate_mfma = router_bwd_mfma(c) ? 1 : 0;
  if (B.gate_mfma) {
    // router weight gradient on the weight-gradient kernel: token slices of at
    // least 128 rows, about 256 blocks in all, each slice's two planes (hi and
    // lo parts of dlogits) [2E][d] float32
    const int64_t per_slice = (2 * E / 128) * (d / 128) / wgrad_run((int)(d / 128));
    int64_t sl = per_slice > 0 ? 256 / per_slice : 1;
    if (sl > T / 128) sl = T / 128;
    B.gate_slices = (int)(sl < 1 ? 1 : sl);
    B.gate_partial = take((size_t)B.gate_slices * 2 * E * d * 4);
    B.dlp = take((size_t)(T * 2 * E * 2));
    B.xr = take((size_t)(T * d * 4));
    B.gso = take((size_t)(B.gate_slices + 1) * 4);
  } else {
    B.gate_partial = take((size_t)B.gate_slices * E * d * 4);
  }
  B.rest_bytes = rest_partial_bytes(c, 1);
  B.rest_partial = take(B.rest_bytes);
  B.total = off;
  return B;
}

static int validate(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->reserved != 0) return MOE_ERR_INVALID_ARG;
  if (c->tokens < 0 || c->d_model <= 0 || c->d_ff <= 0) return MOE_ERR_INVALID_ARG;
  if (c->num_experts < 1 || c->num_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  if (c->top_k < 1 || c->top_k > MOE_MAX_TOP_K || c->top_k > c->num_experts)
    return MOE_ERR_INVALID_ARG;
  if (c->num_shared_experts < 0 || c->num_shared_experts > 1) return MOE_ERR_INVALID_ARG;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID)
    return MOE_ERR_INVALID_ARG;
  if (c->activation < MOE_ACT_GELU || c->activation > MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if ((c->has_bias | c->has_gate_bias | c->drop_tokens) & ~1) return MOE_ERR_INVALID_ARG;
  if ((c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) ||
      (c->router_dtype != MOE_F32 && c->router_dtype != MOE_BF16))
    return MOE_ERR_INVALID_ARG;
  if (c->drop_tokens) {
    const double cf = c->capacity_factor;
    if (!(cf >= 1e-9 && cf <= 1e6)) return MOE_ERR_INVALID_ARG;  // also rejects NaN
    if (c->min_capacity < 0) return MOE_ERR_INVALID_ARG;
  }
  // Sizes this library runs: 32-bit row indices, 16-byte row vectors, and the
  // MFMA tile multiples of the bf16 expert GEMM.
  const int64_t rows = c->tokens * c->top_k + (int64_t)c->num_shared_experts * c->tokens;
  if (c->tokens > (int64_t)1 << 28 || rows >= ((int64_t)1 << 31) - 4096) return MOE_ERR_UNSUPPORTED;
  if (c->d_model > (1 << 20) || c->d_ff > (1 << 20)) return MOE_ERR_UNSUPPORTED;
  if (c->d_model % 8 || c->d_ff % 8) return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == MOE_BF16 && (c->d_model % kGemmAlign || c->d_ff % kGemmAlign))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// ceil(cf * k * T / E) with cf taken at its exact binary value, at least
// min_capacity; -1 when dropping is off.
static int64_t capacity_exact(const moe_config& c) {
  if (!c.drop_tokens) return -1;
  int ex = 0;
  const double fr = frexp(c.capacity_factor, &ex);  // cf = fr 2^ex, fr in [0.5, 1)
  const int64_t m = (int64_t)ldexp(fr, 53);          // exact 53-bit integer
  const int sh = 53 - ex;                            // cf = m / 2^sh, sh in [33, 83]
  const __int128 num = (__int128)m * (__int128)(c.tokens * c.top_k);
  const __int128 den = (__int128)c.num_experts << sh;
  const __int128 q = (num + den - 1) / den;
  int64_t cap = q > (__int128)INT64_MAX ? INT64_MAX : (int64_t)q;
  if (cap < c.min_capacity) cap = c.min_capacity;
  return cap;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Workspace of moe_forward_noalloc: static device memory, one copy per GPU. In
// host code `scratch` names a host-side stand-in, not the device address: the
// address is resolved per device with hipGetSymbolAddress and only that
// pointer is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (resolved once per device).
static int scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_ERR_HIP;
    if (sdev != dev) return MOE_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Layers the training forward and the backward run: every layer moe_forward
// runs (the backward's operand offsets stay within 32 bits for the sizes
// validate admits: d_model, d_ff <= 2^20).
static int validate_train(const moe_config* c) { return validate(c); }

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: layer shape not supported by this library";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_size()";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch or runtime call failed";
    default: return "unknown moe status";
  }
}

const char* moe_version(void) { return "moe-mi355x 0.1.0 (gfx950)"; }

int moe_validate_config(const moe_config* cfg) { return validate(cfg); }

int moe_monitoring(const moe_config* cfg, const moe_stats* st, moe_monitor* out) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (!st || !out) return MOE_ERR_INVALID_ARG;
  const int E = cfg->num_experts;
  const int64_t A = cfg->tokens * cfg->top_k;
  int64_t pre = 0, kept = 0;
  int32_t cmax = st->counts_pre[0], cmin = st->counts_pre[0];
  int used = 0;
  for (int e = 0; e < E; ++e) {
    const int32_t cp = st->counts_pre[e], ck = st->counts_kept[e];
    if (cp < 0 || ck < 0 || ck > cp) return MOE_ERR_INVALID_ARG;
    pre += cp;
    kept += ck;
    cmax = std::max(cmax, cp);
    cmin = std::min(cmin, cp);
    used += ck > 0;
  }
  if (pre != A || (int64_t)st->dropped != A - kept) return MOE_ERR_INVALID_ARG;
  moe_monitor m;
  m.max_count = cmax;
  m.min_count = cmin;
  m.load_imbalance = cmin > 0 ? (double)cmax / (double)cmin : (double)INFINITY;
  m.utilization_rate = (double)used / (double)E;
  m.drop_rate = A > 0 ? (double)st->dropped / (double)A : 0.0;
  *out = m;
  return MOE_OK;
}

int moe_packed_weights_size(const moe_config* cfg, size_t* up_bytes, size_t* down_bytes) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (!up_bytes || !down_bytes) return MOE_ERR_INVALID_ARG;
  if (cfg->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  *up_bytes = packed_weights_bytes(*cfg, 0);
  *down_bytes = packed_weights_bytes(*cfg, 1);
  return MOE_OK;
}

int moe_pack_weights(const moe_config* cfg, const moe_weights* w, void* up_packed,
                     void* down_packed, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!w) return MOE_ERR_INVALID_ARG;
  const bool swiglu = cfg->activation == MOE_ACT_SWIGLU, shared = cfg->num_shared_experts == 1;
  if (up_packed && (!w->w1 || (swiglu && !w->w3) || (shared && (!w->ws1 || (swiglu && !w->ws3)))))
    return MOE_ERR_INVALID_ARG;
  if (down_packed && (!w->w2 || (shared && !w->ws2))) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_pack_weights(*cfg, *w, up_packed, down_packed, (hipStream_t)stream));
}

int moe_capacity(const moe_config* cfg, int64_t* capacity_out) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (!capacity_out) return MOE_ERR_INVALID_ARG;
  *capacity_out = capacity_exact(*cfg);
  return MOE_OK;
}

int moe_workspace_size(const moe_config* cfg, size_t* bytes_out) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (!bytes_out) return MOE_ERR_INVALID_ARG;
  *bytes_out = workspace_layout(*cfg).total;
  return MOE_OK;
}

int moe_route(const moe_config* cfg, const void* x, const void* w_gate, const float* b_gate,
              const float* e_bias, float* logits, int32_t* topk_idx, float* topk_gate,
              moe_stats* stats, void* workspace, size_t workspace_bytes, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!x || !w_gate || !topk_idx || !topk_gate || !stats || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (cfg->has_gate_bias && !b_gate) return MOE_ERR_INVALID_ARG;
  const WsLayout L = workspace_layout(*cfg);
  if (workspace_bytes < L.end_route) return MOE_ERR_WORKSPACE;
  return hip_status(launch_route(*cfg, L, x, w_gate, b_gate, e_bias, logits, topk_idx, topk_gate,
                                 stats, (char*)workspace, (hipStream_t)stream));
}

int moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                int32_t* expert_offsets, int32_t* row_token, int32_t* assign_row, void* x_perm,
                moe_stats* stats, void* workspace, size_t workspace_bytes, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!topk_idx || !expert_offsets || !row_token || !assign_row || !stats || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (x_perm && !x) return MOE_ERR_INVALID_ARG;
  const WsLayout L = workspace_layout(*cfg);
  if (workspace_bytes < L.end_permute) return MOE_ERR_WORKSPACE;
  return hip_status(launch_permute(*cfg, L, capacity_exact(*cfg), topk_idx, x, expert_offsets,
                                   row_token, assign_row, x_perm, stats, (char*)workspace,
                                   (hipStream_t)stream));
}

static int check_weights(const moe_config* c, const void* w1, const void* w3, const float* b1,
                         const void* w2, const float* b2, const void* ws1, const void* ws3,
                         const float* bs1, const void* ws2, const float* bs2) {
  const bool swiglu = c->activation == MOE_ACT_SWIGLU;
  if (!w1 || !w2 || (swiglu && !w3)) return MOE_ERR_INVALID_ARG;
  if (c->has_bias && (!b1 || !b2)) return MOE_ERR_INVALID_ARG;
  if (c->num_shared_experts) {
    if (!ws1 || !ws2 || (swiglu && !ws3)) return MOE_ERR_INVALID_ARG;
    if (c->has_bias && (!bs1 || !bs2)) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

int moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                   const void* w1, const void* w3, const float* b1, const void* w2,
                   const float* b2, const void* ws1, const void* ws3, const float* bs1,
                   const void* ws2, const float* bs2, void* y_perm, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!x_perm || !expert_offsets || !y_perm || !workspace) return MOE_ERR_INVALID_ARG;
  const int wv = check_weights(cfg, w1, w3, b1, w2, b2, ws1, ws3, bs1, ws2, bs2);
  if (wv != MOE_OK) return wv;
  const WsLayout L = workspace_layout(*cfg);
  if (workspace_bytes < L.end_ffn) return MOE_ERR_WORKSPACE;
  const ExpertWeights w{w1, w3, w2, b1, b2, ws1, ws3, ws2, bs1, bs2};
  void* h = (char*)workspace + L.h;
  const hipError_t e = launch_expert_up(*cfg, x_perm, expert_offsets, w, h, (hipStream_t)stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_expert_down(*cfg, h, expert_offsets, w, y_perm, (hipStream_t)stream,
                                       (char*)workspace + L.rest_partial, L.rest_bytes));
}

int moe_expert_up(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                  const void* w1, const void* w3, const float* b1, const void* ws1,
                  const void* ws3, const float* bs1, void* h, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!x_perm || !expert_offsets || !h) return MOE_ERR_INVALID_ARG;
  const bool swiglu = cfg->activation == MOE_ACT_SWIGLU;
  if (!w1 || (swiglu && !w3) || (cfg->has_bias && !b1)) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared_experts && (!ws1 || (swiglu && !ws3) || (cfg->has_bias && !bs1)))
    return MOE_ERR_INVALID_ARG;
  const ExpertWeights w{w1, w3, nullptr, b1, nullptr, ws1, ws3, nullptr, bs1, nullptr};
  return hip_status(launch_expert_up(*cfg, x_perm, expert_offsets, w, h, (hipStream_t)stream));
}

int moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                    const void* w2, const float* b2, const void* ws2, const float* bs2,
                    void* y_perm, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!h || !expert_offsets || !y_perm || !w2 || (cfg->has_bias && !b2)) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared_experts && (!ws2 || (cfg->has_bias && !bs2))) return MOE_ERR_INVALID_ARG;
  const ExpertWeights w{nullptr, nullptr, w2, nullptr, b2, nullptr, nullptr, ws2, nullptr, bs2};
  return hip_status(launch_expert_down(*cfg, h, expert_offsets, w, y_perm, (hipStream_t)stream));
}

int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* expert_offsets,
                const int32_t* assign_row, const float* topk_gate, void* y, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!y_perm || !assign_row || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared_experts && !expert_offsets) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(*cfg, y_perm, expert_offsets, assign_row, topk_gate, y,
                                   (hipStream_t)stream));
}

int moe_forward(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                const moe_routing* r, moe_stats* stats, void* workspace, size_t workspace_bytes,
                void* stream) {
  return moe_forward_profiled(cfg, x, w, y, r, stats, workspace, workspace_bytes, stream, nullptr);
}

int moe_forward_profiled(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                         const moe_routing* r, moe_stats* stats, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!x || !w || !y || !r || !stats || !workspace) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || (cfg->has_gate_bias && !w->b_gate)) return MOE_ERR_INVALID_ARG;
  if (!r->topk_idx || !r->topk_gate || !r->expert_offsets || !r->row_token || !r->assign_row)
    return MOE_ERR_INVALID_ARG;
  const int wv = check_weights(cfg, w->w1, w->w3, w->b1, w->w2, w->b2, w->ws1, w->ws3, w->bs1,
                               w->ws2, w->bs2);
  if (wv != MOE_OK) return wv;
  const WsLayout L = workspace_layout(*cfg);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  const hipStream_t s = (hipStream_t)stream;
  auto mark = [&](int i) {
    return events && events[i] ? hipEventRecord((hipEvent_t)events[i], s) : hipSuccess;
  };
  if (mark(MOE_EV_START) != hipSuccess) return MOE_ERR_HIP;
  // (the reduction of the router statistics runs inside the dispatch's first
  // launch)
  int route_blocks = 0;
  hipError_t e = launch_route(*cfg, L, x, w->w_gate, w->b_gate, w->e_bias, r->logits, r->topk_idx,
                              r->topk_gate, stats, ws, s, &route_blocks);
  if (e != hipSuccess || mark(MOE_EV_ROUTED) != hipSuccess) return MOE_ERR_HIP;
  void* y_perm = ws + L.y_perm;
  // the expert-sorted token rows are not copied: GEMM 1 gathers them from x
  // through row_token
  e = launch_permute(*cfg, L, capacity_exact(*cfg), r->topk_idx, x, r->expert_offsets,
                     r->row_token, r->assign_row, nullptr, stats, ws, s, route_blocks);
  if (e != hipSuccess || mark(MOE_EV_DISPATCHED) != hipSuccess) return MOE_ERR_HIP;
  const ExpertWeights ew{w->w1,  w->w3,  w->w2,  w->b1,  w->b2,        w->ws1,
                         w->ws3, w->ws2, w->bs1, w->bs2, w->up_packed, w->down_packed};
  void* h = ws + L.h;
  e = launch_expert_up(*cfg, x, r->expert_offsets, ew, h, s, r->row_token);
  if (e != hipSuccess || mark(MOE_EV_UP) != hipSuccess) return MOE_ERR_HIP;
  e = launch_expert_down(*cfg, h, r->expert_offsets, ew, y_perm, s, ws + L.rest_partial,
                         L.rest_bytes);
  if (e != hipSuccess || mark(MOE_EV_DOWN) != hipSuccess) return MOE_ERR_HIP;
  e = launch_combine(*cfg, y_perm, r->expert_offsets, r->assign_row, r->topk_gate, y, s);
  if (e != hipSuccess || mark(MOE_EV_END) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_forward_noalloc(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                        const moe_routing* r, moe_stats* stats, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  const size_t need = workspace_layout(*cfg).total;
  if (need > MOE_NOALLOC_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE;
  if (cfg->tokens == 0) return MOE_OK;
  void* ws = nullptr;
  const int st = scratch_of_current_device((hipStream_t)stream, &ws);
  if (st != MOE_OK) return st;
  return moe_forward_profiled(cfg, x, w, y, r, stats, ws, need, stream, nullptr);
}

int moe_update_selection_bias(const moe_config* cfg, const moe_stats* stats, float* e_bias,
                              float gamma, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (!stats || !e_bias) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_bias_update(*cfg, stats, e_bias, gamma, (hipStream_t)stream));
}

int moe_route_hash(const moe_config* cfg, const int32_t* token_ids, const int32_t* table,
                   int64_t table_size, int32_t* topk_idx, float* topk_gate, moe_stats* stats,
                   void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->top_k != 1) return MOE_ERR_UNSUPPORTED;
  if (cfg->tokens == 0) return MOE_OK;
  if (!token_ids || !table || table_size <= 0 || !topk_idx || !topk_gate || !stats)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_hash_route(*cfg, token_ids, table, table_size, topk_idx, topk_gate,
                                      stats, (hipStream_t)stream));
}

int moe_forward_hash(const moe_config* cfg, const void* x, const int32_t* token_ids,
                     const int32_t* table, int64_t table_size, const moe_weights* w, void* y,
                     const moe_routing* r, moe_stats* stats, void* workspace,
                     size_t workspace_bytes, void* stream) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (cfg->top_k != 1) return MOE_ERR_UNSUPPORTED;
  if (cfg->tokens == 0) return MOE_OK;
  if (!x || !token_ids || !table || table_size <= 0 || !w || !y || !r || !stats || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!r->topk_idx || !r->topk_gate || !r->expert_offsets || !r->row_token || !r->assign_row)
    return MOE_ERR_INVALID_ARG;
  const int wv = check_weights(cfg, w->w1, w->w3, w->b1, w->w2, w->b2, w->ws1, w->ws3, w->bs1,
                               w->ws2, w->bs2);
  if (wv != MOE_OK) return wv;
  const WsLayout L = workspace_layout(*cfg);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_hash_route(*cfg, token_ids, table, table_size, r->topk_idx, r->topk_gate,
                                   stats, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_permute(*cfg, L, capacity_exact(*cfg), r->topk_idx, x, r->expert_offsets,
                     r->row_token, r->assign_row, nullptr, stats, ws, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const ExpertWeights ew{w->w1,  w->w3,  w->w2,  w->b1,  w->b2,        w->ws1,
                         w->ws3, w->ws2, w->bs1, w->bs2, w->up_packed, w->down_packed};
  void* h = ws + L.h;
  e = launch_expert_up(*cfg, x, r->expert_offsets, ew, h, s, r->row_token);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_expert_down(*cfg, h, r->expert_offsets, ew, ws + L.y_perm, s, ws + L.rest_partial,
                         L.rest_bytes);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_combine(*cfg, ws + L.y_perm, r->expert_offsets, r->assign_row,
                                   r->topk_gate, y, s));
}

int moe_expert_choice_capacity(const moe_config* cfg, int64_t* capacity_out) {
  const int v = validate(cfg);
  if (v != MOE_OK) return v;
  if (!capacity_out) return MOE_ERR_INVALID_ARG;
  *capacity_out = expert_choice_capacity(*cfg, capacity_exact(*cfg));
  return MOE_OK;
}

static int validate_ec(const moe_config* c) {
  const int v = validate(c);
  if (v != MOE_OK) return v;
  // expert rows E C + S T addressed with 32-bit row indices
  const int64_t C = expert_choice_capacity(*c, capacity_exact(*c));
  if ((int64_t)c->num_experts * C + (int64_t)c->num_shared_experts * c->tokens >=
      ((int64_t)1 << 31) - 4096)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int moe_expert_choice_workspace_size(const moe_config* cfg, size_t* bytes_out) {
  const int v = validate_ec(cfg);
  if (v != MOE_OK) return v;
  if (!bytes_out) return MOE_ERR_INVALID_ARG;
  *bytes_out = expert_choice_layout(*cfg, expert_choice_capacity(*cfg, capacity_exact(*cfg))).total;
  return MOE_OK;
}

int moe_forward_expert_choice(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                              const moe_ec_routing* r, moe_stats* stats, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const int v = validate_ec(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!x || !w || !y || !r || !stats || !workspace) return MOE_ERR_INVALID_ARG;
  if (!r->tokens || !r->gates || !r->token_row) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || (cfg->has_gate_bias && !w->b_gate)) return MOE_ERR_INVALID_ARG;
  const int wv = check_weights(cfg, w->w1, w->w3, w->b1, w->w2, w->b2, w->ws1, w->ws3, w->bs1,
                               w->ws2, w->bs2);
  if (wv != MOE_OK) return wv;
  const int64_t C = expert_choice_capacity(*cfg, capacity_exact(*cfg));
  const EcLayout L = expert_choice_layout(*cfg, C);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  return hip_status(launch_expert_choice_forward(*cfg, L, C, x, *w, y, *r, stats,
                                                 (char*)workspace, (hipStream_t)stream));
}

int moe_forward_train(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                      const moe_routing* r, moe_stats* stats, const moe_saved* saved,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const int v = validate_train(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!x || !w || !y || !r || !stats || !saved || !workspace) return MOE_ERR_INVALID_ARG;
  if (!saved->z || !saved->y_perm || !saved->h) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || (cfg->has_gate_bias && !w->b_gate)) return MOE_ERR_INVALID_ARG;
  if (!r->logits || !r->topk_idx || !r->topk_gate || !r->expert_offsets || !r->row_token ||
      !r->assign_row)
    return MOE_ERR_INVALID_ARG;
  const int wv = check_weights(cfg, w->w1, w->w3, w->b1, w->w2, w->b2, w->ws1, w->ws3, w->bs1,
                               w->ws2, w->bs2);
  if (wv != MOE_OK) return wv;
  const WsLayout L = workspace_layout(*cfg);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  const hipStream_t s = (hipStream_t)stream;
  int route_blocks = 0;
  hipError_t e = launch_route(*cfg, L, x, w->w_gate, w->b_gate, w->e_bias, r->logits, r->topk_idx,
                              r->topk_gate, stats, ws, s, &route_blocks);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_permute(*cfg, L, capacity_exact(*cfg), r->topk_idx, x, r->expert_offsets,
                     r->row_token, r->assign_row, nullptr, stats, ws, s, route_blocks);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const ExpertWeights ew{w->w1, w->w3, w->w2, w->b1, w->b2, w->ws1, w->ws3, w->ws2, w->bs1, w->bs2};
  e = launch_expert_up_linear(*cfg, x, r->expert_offsets, ew, saved->z, s, r->row_token);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_act_rows(*cfg, saved->z, r->expert_offsets, saved->h, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_expert_down(*cfg, saved->h, r->expert_offsets, ew, saved->y_perm, s,
                         ws + L.rest_partial, L.rest_bytes);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_combine(*cfg, saved->y_perm, r->expert_offsets, r->assign_row, r->topk_gate, y, s);
  return hip_status(e);
}

int moe_backward_workspace_size(const moe_config* cfg, size_t* bytes_out) {
  const int v = validate_train(cfg);
  if (v != MOE_OK) return v;
  if (!bytes_out) return MOE_ERR_INVALID_ARG;
  *bytes_out = (cfg->act_dtype == MOE_BF16 ? backward_layout(*cfg) : backward_layout_f32(*cfg)).total;
  return MOE_OK;
}

int moe_backward(const moe_config* cfg, const void* x, const moe_weights* w, const moe_routing* r,
                 const moe_stats* stats, const moe_saved* saved, const void* dy, float aux_coef,
                 float z_coef, const moe_grads* g, void* workspace, size_t workspace_bytes,
                 void* stream) {
  const int v = validate_train(cfg);
  if (v != MOE_OK) return v;
  if (cfg->tokens == 0) return MOE_OK;
  if (!x || !w || !r || !stats || !saved || !dy || !g || !workspace) return MOE_ERR_INVALID_ARG;
  if (!saved->z || !saved->y_perm || !saved->h) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || !w->w1 || !w->w2) return MOE_ERR_INVALID_ARG;
  if (!r->logits || !r->topk_idx || !r->topk_gate || !r->expert_offsets || !r->row_token ||
      !r->assign_row)
    return MOE_ERR_INVALID_ARG;
  const bool shared = cfg->num_shared_experts == 1, bias = cfg->has_bias != 0;
  if (shared && (!w->ws1 || !w->ws2)) return MOE_ERR_INVALID_ARG;
  if (!g->dx || !g->dw_gate || !g->dw1 || !g->dw2) return MOE_ERR_INVALID_ARG;
  if (cfg->has_gate_bias && !g->db_gate) return MOE_ERR_INVALID_ARG;
  if (bias && (!g->db1 || !g->db2)) return MOE_ERR_INVALID_ARG;
  if (shared && (!g->dws1 || !g->dws2 || (bias && (!g->dbs1 || !g->dbs2))))
    return MOE_ERR_INVALID_ARG;
  const bool swiglu = cfg->activation == MOE_ACT_SWIGLU;
  if (swiglu && (!w->w3 || !g->dw3 || (shared && (!w->ws3 || !g->dws3)))) return MOE_ERR_INVALID_ARG;
  const BwdLayout B = cfg->act_dtype == MOE_BF16 ? backward_layout(*cfg) : backward_layout_f32(*cfg);
  if (workspace_bytes < B.total) return MOE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  const hipStream_t s = (hipStream_t)stream;
  if (cfg->act_dtype != MOE_BF16)
    return hip_status(launch_backward_f32(*cfg, B, x, *w, *r, stats, *saved, dy, aux_coef, z_coef,
                                          *g, ws, s));
  hipError_t e = launch_backward_misc(*cfg, B, x, *w, *r, stats, *saved, dy, aux_coef, z_coef, *g,
                                      ws, s, 0);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // GELU / ReLU with biases: the dZ GEMM also writes the column sums of its tiles
  e = launch_backward_dz(*cfg, ws + B.dyp, r->expert_offsets, w->w2, w->ws2, saved->z,
                         ws + (swiglu ? B.dh : B.dz),
                         cfg->has_bias && !swiglu ? (float*)(ws + B.colsum1) : nullptr,
                         (int)(B.ldk / 64), s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (swiglu) {
    e = launch_dswiglu(*cfg, ws + B.dh, saved->z, ws + B.dz, r->expert_offsets, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  e = launch_backward_dx(*cfg, ws + B.dz, r->expert_offsets, w->w1, w->w3, w->ws1, w->ws3,
                         ws + B.dxp, s, ws + B.rest_partial, B.rest_bytes);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_backward_misc(*cfg, B, x, *w, *r, stats, *saved, dy, aux_coef, z_coef,
                                         *g, ws, s, 1));
}

}  // extern "C"
