/*
 * moe.h — C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward.
 *
 * The layer (token-choice top-k routing):
 *   h = x . W_g^T (+ b_g)                       router logits, float32
 *   p = softmax(h)   or   s = sigmoid(h)         score function, float32
 *   top-k experts per token by key (h for softmax, s + e_bias for sigmoid),
 *   gates renormalised over the k selected (unbiased) scores
 *   capacity-limited dispatch into an expert-sorted row buffer
 *   E_e(x) = W2[e] act(W1[e] x + b1[e]) + b2[e]    (SwiGLU: W2[e](silu(W1 x) * W3 x))
 *   y[t] = sum_j kept(t,j) g[t,j] E_{i_j}(x_t)  (+ shared expert E_s(x_t))
 *   L_aux = E sum_i f_i P_i,   z = mean_t logsumexp(h_t)^2
 *
 * Sources (web pages on sparse Mixture-of-Experts):
 *   [P1] "MoE Training: Mixture of Experts" (claudewave skill page): "Basic MoE
 *        Architecture", "2. Routing Mechanisms", "3. Load Balancing".
 *   [P2] "MoE Training Guide" (DeepSpeed-based guide): "Basic MoE Configuration",
 *        "Core MoE Parameters" items 4-7, "Monitoring".
 *   [P3] "moe_code.py" (Mixture of Experts: Complete Implementation): classes
 *        Expert, Router, MixtureOfExperts, SwitchMoE.
 *   [P4] "Mixture of Experts (MoE) From Scratch to DeepSeek V3" (CS336 lecture 4
 *        notes): token-choice top-k formula, auxiliary loss, auxiliary-loss-free
 *        bias, token dropping, router precision and z-loss, V3 sigmoid routing,
 *        shared + fine-grained experts.
 *   [P5] "Moe(Mixtrue of Experts)" survey: Mixtral parameter count.
 *
 * Conventions for every entry point:
 *   - Pointers named x, w*, b*, logits, topk_*, expert_offsets, row_token,
 *     assign_row, x_perm, y_perm, y, stats and workspace are DEVICE pointers; cfg
 *     and the structs passed by pointer are HOST memory. The caller owns every
 *     buffer; the library allocates nothing and keeps no state between calls,
 *     except two kinds of static device memory per GPU, both reserved when the
 *     library is loaded: the work-queue counters of the weight-streaming GEMM
 *     (256 slots of 1 KB, taken in turn by its launches and left at zero by
 *     each; calls on different streams may run at the same time as long as
 *     fewer than 256 such launches are in flight at once) and the workspace of
 *     moe_forward_noalloc.
 *   - stream is a hipStream_t passed as void*; NULL means the default stream.
 *     All device work is enqueued on it asynchronously; no entry point
 *     synchronises. Host-only helpers do no device work at all.
 *   - Tensors are dense row-major. Weights use the nn.Linear [out, in] layout,
 *     stacked on a leading expert axis: W1, W3 [E, d_ff, d_model], W2
 *     [E, d_model, d_ff], so both operands of every product are contiguous
 *     along the reduction axis.
 *   - Element types: activations, x, W1, W3, W2 and every row buffer have type
 *     act_dtype; W_g has router_dtype; biases, logits, gates and statistics are
 *     float32; indices are int32.
 *   - Return value: MOE_OK or an error code. Arguments are validated before any
 *     launch; on error nothing is enqueued. A failed launch returns MOE_ERR_HIP.
 *     Entry points never abort, throw or print. Non-finite inputs give
 *     unspecified (but memory-safe) results.
 *   - tokens == 0 is a valid no-op: nothing is enqueued and nothing written.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOP_K 8

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, out-of-range field, inconsistent sizes */
  MOE_ERR_UNSUPPORTED = 2, /* valid layer this library does not run (shape multiple) */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
};

enum moe_score_fn { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum moe_activation { MOE_ACT_GELU = 0, MOE_ACT_RELU = 1, MOE_ACT_SWIGLU = 2 };
enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

/*
 * Layer configuration (host struct). Field names follow the DeepSpeed MoE keys
 * of [P2] "Basic MoE Configuration" / "Core MoE Parameters" and the module
 * arguments of [P1] MoELayer(hidden_size, num_experts, top_k) and [P3]
 * MixtureOfExperts(d_model, d_ff, num_experts, top_k).
 */
typedef struct moe_config {
  int64_t tokens;             /* T = batch * sequence, >= 0                         */
  int64_t d_model;            /* hidden size d, a multiple of 8                       */
  int64_t d_ff;               /* expert inner size F, a multiple of 8                 */
  int32_t num_experts;        /* routed experts E, 1..256                             */
  int32_t top_k;              /* k, 1..min(E, 8)                                      */
  int32_t num_shared_experts; /* 0 or 1: always-active expert with gate 1 [P4]       */
  int32_t score_fn;           /* MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID               */
  int32_t activation;         /* MOE_ACT_GELU (exact erf), MOE_ACT_RELU, MOE_ACT_SWIGLU */
  int32_t has_bias;           /* experts carry b1 [E,F] and b2 [E,d]                  */
  int32_t has_gate_bias;      /* router carries b_g [E]                               */
  int32_t drop_tokens;        /* 0: no capacity limit ([P2] item 7)                   */
  int32_t min_capacity;       /* >= 0 ([P2] item 6)                                   */
  int32_t act_dtype;          /* MOE_F32 or MOE_BF16                                  */
  int32_t router_dtype;       /* dtype of W_g: MOE_F32 or MOE_BF16                    */
  int32_t reserved;           /* must be 0                                            */
  double capacity_factor;     /* > 0 and finite when drop_tokens ([P2] items 4-5)     */
} moe_config;

/*
 * Device-resident statistics written by moe_route (prob_mean, z_loss) and
 * moe_permute (everything else). [P1] "3. Load Balancing"; [P2] "Monitoring";
 * [P3] MixtureOfExperts routing_info / expert usage; [P4] auxiliary loss and
 * z-loss. f_i counts top-k picks before capacity, divided by T*k; for the
 * sigmoid router P_i is the mean of s_ti / sum_e s_te.
 */
typedef struct moe_stats {
  int32_t counts_pre[MOE_MAX_EXPERTS];  /* top-k picks per expert                    */
  int32_t counts_kept[MOE_MAX_EXPERTS]; /* min(counts_pre, capacity)                 */
  float frac[MOE_MAX_EXPERTS];          /* f_i = counts_pre / (T k)                  */
  float prob_mean[MOE_MAX_EXPERTS];     /* P_i                                       */
  float l_aux;                          /* E sum_i f_i P_i                           */
  float z_loss;                         /* mean_t logsumexp(h_t)^2                   */
  int32_t capacity;                     /* per-expert capacity, -1 when unlimited    */
  int32_t kept;                         /* sum counts_kept (= R, the routed rows)    */
  int32_t dropped;                      /* T k - kept                                */
  int32_t reserved[3];
} moe_stats;

/* Weights for moe_forward (device pointers; NULL where the layer has none). */
typedef struct moe_weights {
  const void* w_gate;  /* [E, d] router_dtype                                  */
  const float* b_gate; /* [E] if has_gate_bias, else NULL                      */
  const float* e_bias; /* [E] sigmoid selection bias, or NULL ([P4] V3 bias b_i) */
  const void* w1;      /* [E, F, d]                                            */
  const void* w3;      /* [E, F, d] for SwiGLU, else NULL                      */
  const float* b1;     /* [E, F] if has_bias, else NULL                        */
  const void* w2;      /* [E, d, F]                                            */
  const float* b2;     /* [E, d] if has_bias, else NULL                        */
  const void* ws1;     /* shared expert [F, d] (num_shared_experts == 1)       */
  const void* ws3;     /* shared expert [F, d] for SwiGLU                      */
  const float* bs1;    /* shared expert [F] if has_bias                        */
  const void* ws2;     /* shared expert [d, F]                                 */
  const float* bs2;    /* shared expert [d] if has_bias                        */
  /* Optional packed copies written by moe_pack_weights (NULL: not used). When
   * given, the grouped GEMM reads the weights of groups with few rows from
   * them (same values, the weight-streaming kernel's order); every other read
   * uses w1 / w3 / w2 / ws*. Read by moe_forward, moe_forward_profiled,
   * moe_forward_noalloc and moe_forward_hash; the other entry points ignore them. */
  const void* up_packed;   /* moe_packed_weights_size up_bytes: W1 (and W3) of every group */
  const void* down_packed; /* moe_packed_weights_size down_bytes: W2 of every group        */
} moe_weights;

/* Routing and dispatch results of moe_forward (device buffers the caller owns). */
typedef struct moe_routing {
  float* logits;           /* [T, E] float32, or NULL to skip writing them        */
  int32_t* topk_idx;       /* [T, k]                                              */
  float* topk_gate;        /* [T, k]                                              */
  int32_t* expert_offsets; /* [E + S + 1], S = num_shared_experts                 */
  int32_t* row_token;      /* [T k + S T]                                         */
  int32_t* assign_row;     /* [T, k]                                              */
} moe_routing;

/* Monitoring figures of one routed batch, derived from its statistics. */
typedef struct moe_monitor {
  double load_imbalance;   /* max_i counts_pre / min_i counts_pre; +inf when an expert got no pick */
  double utilization_rate; /* (experts with counts_kept > 0) / E                                    */
  double drop_rate;        /* dropped / (T k); 0 when T = 0                                         */
  int32_t max_count;       /* max_i counts_pre                                                      */
  int32_t min_count;       /* min_i counts_pre                                                      */
} moe_monitor;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(int status);

/* Library version string (static). */
const char* moe_version(void);

/* Host only. MOE_OK if cfg describes a layer this library runs, else the code
 * moe_forward would return for it (MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED). */
int moe_validate_config(const moe_config* cfg);

/*
 * Host only. Bytes of the packed weight copies moe_pack_weights writes, over
 * the E + S groups: up_bytes for GEMM 1's W1 (and W3), down_bytes for GEMM 2's
 * W2 (each the size of the matrices it copies). bf16 layers only
 * (MOE_ERR_UNSUPPORTED for float32 layers).
 */
int moe_packed_weights_size(const moe_config* cfg, size_t* up_bytes, size_t* down_bytes);

/*
 * Copies the expert weights of w (w1, w3, w2 and the shared expert's ws1,
 * ws3, ws2) into up_packed / down_packed (device buffers of the sizes above;
 * either may be NULL to skip it) in the order the weight-streaming grouped
 * GEMM reads them: for each group, slab of 256 weight rows (SwiGLU: 128 rows
 * of W1 with the same rows of W3), 64-deep K step and wave, 8 KB in MFMA
 * fragment order. The values are unchanged; pass the buffers as
 * moe_weights.up_packed / down_packed to forward calls. A one-time conversion
 * for a set of weights (the copy must be redone when the weights change).
 * bf16 layers only. Enqueued on `stream`; returns MOE_ERR_HIP on a failed launch.
 */
int moe_pack_weights(const moe_config* cfg, const moe_weights* w, void* up_packed,
                     void* down_packed, void* stream);

/*
 * Host only. The monitoring figures of [P2] "Monitoring" (the load imbalance as
 * the ratio of the largest to the smallest per-expert count, the utilisation as
 * the share of experts that receive tokens, the drop rate as dropped over total
 * assignments) from a HOST copy of the moe_stats a forward wrote for cfg.
 * Counts are the top-k picks before capacity (counts_pre) for the imbalance and
 * the kept rows (counts_kept) for the utilisation. Reads only the first E
 * entries of the count arrays and `dropped`. Returns MOE_ERR_INVALID_ARG for a
 * NULL pointer, an invalid cfg, or counts that are negative or that contradict
 * the layer (sum counts_pre != T k, counts_kept > counts_pre, dropped !=
 * T k - sum counts_kept); `out` is written only on MOE_OK.
 */
int moe_monitoring(const moe_config* cfg, const moe_stats* host_stats, moe_monitor* out);

/*
 * Host only. Per-expert capacity C = max(min_capacity, ceil(capacity_factor *
 * top_k * tokens / num_experts)), or -1 when drop_tokens == 0.
 * [P2] "Core MoE Parameters" items 4-7 give (tokens / num_experts) x factor and
 * the minimum; this library counts the T*k assignments as "tokens" and rounds
 * up, using the exact binary value of capacity_factor.
 */
int moe_capacity(const moe_config* cfg, int64_t* capacity_out);

/* Host only. Workspace bytes needed by moe_forward (enough for every stage). */
int moe_workspace_size(const moe_config* cfg, size_t* bytes_out);

/*
 * Router, score function, top-k and renormalised gates; writes stats->prob_mean
 * and stats->z_loss.
 * [P4] token-choice formula h(x) = x W_g, p = Softmax(h), TopK; router softmax
 * in float32; [P1] "Basic MoE Architecture" (gate nn.Linear with bias, softmax,
 * topk, renormalise); [P4] V3 sigmoid routing with selection bias b_i.
 *   x         [T, d] act_dtype
 *   w_gate    [E, d] router_dtype;  b_gate [E] or NULL;  e_bias [E] or NULL
 *   logits    [T, E] float32 output, or NULL
 *   topk_idx  [T, k] int32 output: experts in descending key order; equal keys
 *             go to the lower index. Key = h (softmax) or s + e_bias (sigmoid).
 *   topk_gate [T, k] float32 output: p_j / sum_sel p (softmax) or s_j / sum_sel s
 *             (sigmoid, unbiased s)
 *   stats     device moe_stats (prob_mean, z_loss written)
 */
int moe_route(const moe_config* cfg, const void* x, const void* w_gate, const float* b_gate,
              const float* e_bias, float* logits, int32_t* topk_idx, float* topk_gate,
              moe_stats* stats, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Capacity-limited dispatch: histogram, stable expert-sorted order, drop set,
 * and the gather of token rows into the expert-sorted buffer. Completes the
 * statistics (counts, f_i, L_aux from the P_i moe_route wrote, kept, dropped).
 * [P4] "Token Dropping"; [P2] items 4-7. Queue order is k-major then
 * token-ascending: assignment (t, j) has priority j*T + t; it is kept iff its
 * position in its expert's queue is < capacity (always when drop_tokens == 0).
 * Rows are ordered by expert, then queue position. With a shared expert, rows
 * R..R+T-1 (R = kept routed rows) hold every token in order (group E).
 *   topk_idx       [T, k] int32 input (values in [0, E))
 *   x              [T, d] act_dtype
 *   expert_offsets [E + S + 1] int32 output: exclusive scan of kept rows per group
 *   row_token      [T k + S T] int32 output: source token of each row (first
 *                  expert_offsets[E + S] entries written)
 *   assign_row     [T, k] int32 output: row of (t, j) or -1 when dropped
 *   x_perm         [T k + S T, d] act_dtype output (first expert_offsets[E+S]
 *                  rows written), or NULL to skip the gather
 *   stats          device moe_stats (reads prob_mean; writes the rest)
 */
int moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                int32_t* expert_offsets, int32_t* row_token, int32_t* assign_row, void* x_perm,
                moe_stats* stats, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped expert FFN over the expert-sorted rows: for group g (routed expert
 * g < E, shared expert g == E) and rows expert_offsets[g] .. expert_offsets[g+1]-1,
 *   y_perm[r] = W2[g] act(W1[g] x_perm[r] + b1[g]) + b2[g]
 * (SwiGLU: W2[g] (silu(W1[g] x) * (W3[g] x))), float32 accumulation, the
 * intermediate rounded to act_dtype. [P1] expert nn.Sequential(Linear, GELU,
 * Linear); [P3] Expert (ReLU; dropout is the identity in a forward pass); [P5]
 * three matrices per Mixtral expert (SwiGLU).
 *   x_perm         [rows, d] act_dtype, rows = expert_offsets[E + S]
 *   expert_offsets [E + S + 1] int32, non-decreasing, expert_offsets[0] == 0,
 *                  expert_offsets[E + S] <= T k + S T
 *   w1, w3, b1, w2, b2   routed expert weights (w3 only for SwiGLU, b* iff has_bias)
 *   ws1, ws3, bs1, ws2, bs2   shared expert weights (iff num_shared_experts)
 *   y_perm         [rows, d] act_dtype output
 */
int moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                   const void* w1, const void* w3, const float* b1, const void* w2,
                   const float* b2, const void* ws1, const void* ws3, const float* bs1,
                   const void* ws2, const float* bs2, void* y_perm, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * First grouped GEMM of moe_expert_ffn alone, with the activation fused:
 *   h[r] = act(W1[g] x_perm[r] + b1[g])   (SwiGLU: silu(W1[g] x) * (W3[g] x))
 * for the rows r of each group g as in moe_expert_ffn; h is [T k + S T, d_ff]
 * act_dtype (rows beyond expert_offsets[E + S] are not written). Same sources
 * as moe_expert_ffn. Needs no workspace.
 */
int moe_expert_up(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                  const void* w1, const void* w3, const float* b1, const void* ws1,
                  const void* ws3, const float* bs1, void* h, void* stream);

/*
 * Second grouped GEMM of moe_expert_ffn alone: y_perm[r] = W2[g] h[r] + b2[g]
 * for the rows r of each group g. h as written by moe_expert_up; y_perm
 * [T k + S T, d_model] act_dtype. Needs no workspace.
 */
int moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                    const void* w2, const float* b2, const void* ws2, const float* bs2,
                    void* y_perm, void* stream);

/*
 * Gate-weighted combine: y[t] = sum_j [assign_row[t,j] >= 0] topk_gate[t,j] *
 * y_perm[assign_row[t,j]] (+ y_perm[expert_offsets[E] + t] with a shared
 * expert), float32 accumulation in j order, one rounding to act_dtype. A
 * token whose every choice was dropped gets zeros. No residual is added.
 * [P4] y = sum_{i in TopK} Gate_i E_i(x); [P1] "Weighted Combination";
 * [P4] shared experts are always active.
 *   y_perm [rows, d]; expert_offsets [E + S + 1] (read only with a shared expert,
 *   may be NULL otherwise); assign_row, topk_gate [T, k]; y [T, d] output.
 */
int moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* expert_offsets,
                const int32_t* assign_row, const float* topk_gate, void* y, void* stream);

/*
 * The whole layer forward: moe_route, moe_permute, moe_expert_ffn and
 * moe_combine on one stream, with the expert intermediate and outputs kept in
 * the workspace. The expert-sorted copy of the token rows is not made: the
 * first expert GEMM reads token rows of x through routing->row_token, which
 * gives the same results as the staged path bit for bit.
 *   x [T, d] act_dtype;  w: weights;  y [T, d] act_dtype output;
 *   routing: caller buffers for the routing results (logits may be NULL);
 *   stats: device moe_stats;  workspace >= moe_workspace_size(cfg) bytes.
 */
int moe_forward(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                const moe_routing* routing, moe_stats* stats, void* workspace,
                size_t workspace_bytes, void* stream);

/* Stage boundaries moe_forward_profiled marks with events. */
enum {
  MOE_EV_START = 0,     /* before the router                                   */
  MOE_EV_ROUTED = 1,    /* after moe_route's kernels                           */
  MOE_EV_DISPATCHED = 2,/* after moe_permute's kernels                         */
  MOE_EV_UP = 3,        /* after expert GEMM 1 (every group)                   */
  MOE_EV_DOWN = 4,      /* after expert GEMM 2 (every group)                   */
  MOE_EV_END = 5,       /* after the combine                                   */
  MOE_FORWARD_EVENTS = 6
};

/*
 * moe_forward with timing markers, for measuring the stages of the real
 * forward path: the same kernels with the same arguments on the same stream,
 * plus hipEventRecord(events[i], stream) at each boundary i of the enum above.
 *   events  host array of MOE_FORWARD_EVENTS hipEvent_t handles the caller
 *           created (NULL entries are skipped; events itself may be NULL,
 *           which makes the call identical to moe_forward).
 * Returns MOE_ERR_HIP if recording an event fails.
 */
int moe_forward_profiled(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                         const moe_routing* routing, moe_stats* stats, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events);

/* Size of the device buffer moe_forward_noalloc works in (per GPU). */
#define MOE_NOALLOC_WORKSPACE_BYTES ((size_t)128 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward
 * with its workspace taken from a buffer the library holds in static device
 * memory, MOE_NOALLOC_WORKSPACE_BYTES (128 MiB) on each GPU it runs on, kept
 * until the process ends. Same kernels, arguments and results as moe_forward
 * with a caller workspace. Allocates nothing and calls no allocating routine.
 *   The stream must belong to the current device (NULL: its null stream).
 *   Returns MOE_ERR_WORKSPACE if moe_workspace_size(cfg) exceeds the limit
 *   (checked before anything else touches the GPU), MOE_ERR_INVALID_ARG if the
 *   stream belongs to another device.
 *   Every call on one GPU shares that GPU's buffer, and the buffer keeps the
 *   last call's contents (the forward needs no zeroed workspace): calls that
 *   overlap on one GPU (on different streams, or from several threads) race.
 *   The first call on a device resolves the buffer's address (HIP loads the
 *   library's device code there if it has not done so yet): make that first
 *   call outside graph capture.
 */
int moe_forward_noalloc(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                        const moe_routing* routing, moe_stats* stats, void* stream);

/* ------------------------------------------------------------------ balancing, hash routing */

/*
 * One update of the sigmoid router's selection bias ([P4] auxiliary-loss-free
 * balancing: b_i is lowered when expert i is overloaded and raised when it is
 * idle): e_bias[i] -= gamma * sign(c_i E - T k), with c_i = stats->counts_pre[i]
 * (top-k picks before capacity, as moe_permute / moe_forward wrote them) and T k /
 * E the mean load, compared exactly in integers; float32 arithmetic. The step
 * gamma is the caller's (the pages give none).
 *   stats   device moe_stats of the routing step to balance
 *   e_bias  [E] float32 device buffer, updated in place
 */
int moe_update_selection_bias(const moe_config* cfg, const moe_stats* stats, float* e_bias,
                              float gamma, void* stream);

/*
 * Hash routing ([P5] hash-based routing: a token -> expert map fixed in advance
 * replaces the gating network): topk_idx[t] = table[token_ids[t]], topk_gate[t]
 * = 1, for a layer with top_k == 1 (other k: MOE_ERR_UNSUPPORTED). Ids outside
 * [0, table_size) and table entries outside [0, E) are clamped. Writes
 * stats->prob_mean = 0 and stats->z_loss = 0 (no router).
 *   token_ids [T] int32;  table [table_size] int32;  topk_idx, topk_gate [T, 1]
 */
int moe_route_hash(const moe_config* cfg, const int32_t* token_ids, const int32_t* table,
                   int64_t table_size, int32_t* topk_idx, float* topk_gate, moe_stats* stats,
                   void* stream);

/*
 * The layer forward with hash routing: moe_route_hash, then moe_permute,
 * moe_expert_ffn and moe_combine as in moe_forward (capacity applies; the gate
 * weights are not read and may be NULL; routing->logits is not written).
 */
int moe_forward_hash(const moe_config* cfg, const void* x, const int32_t* token_ids,
                     const int32_t* table, int64_t table_size, const moe_weights* w, void* y,
                     const moe_routing* routing, moe_stats* stats, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ expert choice
 * Expert-choice routing ([P1] "2. Routing Mechanisms", expert choice routing;
 * [P4] routing strategies; [P5] expert-choice routing): every expert takes its
 * C best tokens over the transposed [E, T] router scores, so each expert is
 * exactly full, while a token may be served by several experts or by none.
 * Key = the float32 router logit (both score functions increase with it);
 * equal keys go to the lower token. The output of expert e for token t is
 * weighted by the router score g[t, e]: the softmax probability p[t, e] over
 * experts, or with score_fn MOE_SCORE_SIGMOID the sigmoid score
 * 1 / (1 + exp(-h[t, e])) itself ([P4] V3 sigmoid routing; a token has
 * no fixed number of picks, so there is no renormalisation, and the selection
 * bias e_bias, a per-expert constant, cannot change an expert's choice and is
 * not read). y[t] = sum over the experts that chose t of g[t, e] E_e(x_t)
 * (+ the shared expert). C = max(min_capacity, ceil(capacity_factor k T / E))
 * (ceil(k T / E) when drop_tokens == 0), at most T.
 */

/* Expert-choice routing results (device buffers the caller owns). */
typedef struct moe_ec_routing {
  float* logits;      /* [T, E] float32, or NULL                                        */
  int32_t* tokens;    /* [E, C]: expert e's chosen tokens, ascending (rows e C .. e C+C-1) */
  float* gates;       /* [E, C]: g[t, e] of those tokens (p, or the sigmoid score)       */
  int32_t* token_row; /* [T, E]: row of (t, e), or -1 when expert e did not choose t     */
} moe_ec_routing;

/* Host only. Tokens per expert C of expert-choice routing. */
int moe_expert_choice_capacity(const moe_config* cfg, int64_t* capacity_out);

/* Host only. Workspace bytes needed by moe_forward_expert_choice. */
int moe_expert_choice_workspace_size(const moe_config* cfg, size_t* bytes_out);

/*
 * The layer forward with expert-choice routing on one stream: router logits,
 * per-expert top-C selection, the grouped GEMMs of moe_forward on the E C rows
 * (+ T shared rows), and the gate-weighted combine. stats: counts_pre =
 * counts_kept = C, f_i = 1/E, P_i and z as for token choice (P_i the mean of
 * p[t, i], or of s[t, i] / sum_e s[t, e] for the sigmoid router), L_aux =
 * E sum f_i P_i, capacity = C, kept = E C, dropped = the number of tokens no
 * expert chose.
 *   x [T, d];  w: weights (e_bias unused);  y [T, d] output;  r: routing buffers;
 *   stats: device moe_stats;  workspace >= moe_expert_choice_workspace_size(cfg).
 */
int moe_forward_expert_choice(const moe_config* cfg, const void* x, const moe_weights* w,
                              void* y, const moe_ec_routing* r, moe_stats* stats,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ training
 * The layer's backward pass. The objective differentiated is
 *   L = <dy, y> + aux_coef * L_aux + z_coef * z
 * where dy is the gradient of the caller's loss with respect to the layer output
 * and aux_coef, z_coef the weights of the balance loss and the router z-loss in
 * that loss ([P1] "3. Load Balancing": the auxiliary loss is added to the task
 * loss with a small coefficient; [P4] router z-loss). The top-k choices, the
 * capacity decisions and the counts f_i are piecewise constant and carry no
 * gradient; the sigmoid selection bias e_bias receives none.
 * Both layer types run it, with GELU, ReLU or SwiGLU experts: bf16 layers on
 * the MFMA GEMMs, float32 layers in float32 throughout (plain kernels, one
 * output per thread).
 */

/* Forward activations the backward reads (device buffers the caller owns). */
typedef struct moe_saved {
  void* z;      /* [T k + S T, F] act_dtype: W1 x + b1 per expert-sorted row;
                   SwiGLU: [2, T k + S T, F], the planes W1 x + b1 and W3 x       */
  void* y_perm; /* [T k + S T, d] act_dtype: the expert outputs E_e(x) per row  */
  void* h;      /* [T k + S T, F] act_dtype: act(z) per row (SwiGLU: silu(z1) u),
                   the input of the second expert GEMM                           */
} moe_saved;

/* Gradients written by moe_backward (device buffers; float32 except dx). Every
 * buffer is overwritten (not accumulated into). NULL where the layer has no such
 * parameter: db_gate iff has_gate_bias, db1/db2 iff has_bias, the ws* ones iff
 * num_shared_experts, dw3 / dws3 iff SwiGLU. */
typedef struct moe_grads {
  void* dx;        /* [T, d] act_dtype                         */
  float* dw_gate;  /* [E, d]                                   */
  float* db_gate;  /* [E]                                      */
  float* dw1;      /* [E, F, d]                                */
  float* db1;      /* [E, F]                                   */
  float* dw2;      /* [E, d, F]                                */
  float* db2;      /* [E, d]                                   */
  float* dws1;     /* [F, d]   shared expert                   */
  float* dbs1;     /* [F]                                      */
  float* dws2;     /* [d, F]                                   */
  float* dbs2;     /* [d]                                      */
  float* dw3;      /* [E, F, d]  SwiGLU only                   */
  float* dws3;     /* [F, d]     SwiGLU with a shared expert   */
} moe_grads;

/*
 * The layer forward of moe_forward that also keeps what the backward needs:
 * routing->logits (required here) and saved->z, saved->y_perm, saved->h (every
 * saved buffer required). The expert activation is applied to z after its
 * rounding to act_dtype and h is kept as rounded, so the backward uses exactly
 * the h the second GEMM read (SwiGLU: h = silu(z1) u from the two rounded
 * planes). Same arguments and workspace as moe_forward.
 */
int moe_forward_train(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                      const moe_routing* routing, moe_stats* stats, const moe_saved* saved,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Host only. Workspace bytes needed by moe_backward. */
int moe_backward_workspace_size(const moe_config* cfg, size_t* bytes_out);

/*
 * Gradients of the objective above for one layer, from the results of
 * moe_forward_train on the same x and weights (routing, stats and saved must be
 * unchanged since). Chain rule through combine ([P4] y = sum Gate_i E_i(x)), the
 * expert FFN ([P1] "Basic MoE Architecture"), the renormalised top-k gates and
 * the score function ([P1] "Basic MoE Architecture", [P4] V3 sigmoid routing),
 * L_aux ([P1] "3. Load Balancing") and the z-loss ([P4]), and the gate linear
 * layer. bf16 layers: expert GEMMs in bf16 with float32 accumulation; router
 * math, weight and bias gradients in float32. float32 layers: float32 for every
 * step. Deterministic (no floating-point atomics).
 *   x, w         the forward's inputs;  routing, stats, saved: the forward's outputs
 *   dy           [T, d] act_dtype
 *   grads        output buffers (moe_grads)
 *   workspace    >= moe_backward_workspace_size(cfg) bytes
 */
int moe_backward(const moe_config* cfg, const void* x, const moe_weights* w,
                 const moe_routing* routing, const moe_stats* stats, const moe_saved* saved,
                 const void* dy, float aux_coef, float z_coef, const moe_grads* grads,
                 void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
