"""CPU oracle for the sparse Mixture-of-Experts layer forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test-suite, the smoke check of the package entry
file and the CPU-baseline leg of the benchmark use it. It shares no code with
the HIP library; both receive the same seeded inputs from the input generator.

Plain numpy. Arithmetic is float64, except where the pages fix the precision:
the router's softmax is taken in float32 (MoE From Scratch to DeepSeek V3,
stability tricks, router precision; the Moe(Mixtrue of Experts) survey gives
the same advice in its stability section), so router logits are
float32 values and the top-k decision is taken on float32 keys. Library
primitives used as steps: matrix product, stable argsort, bincount, erf.

What is computed (one MoE layer forward, token choice):
  h(x) = x . W_g (+ b_g)                       router logits
  p = softmax(h)  or  s = sigmoid(h)           score function
  top-k by key, gates renormalised over the k selected scores
  capacity-limited dispatch in k-major, token-ascending queue order
  E_e(x) = W2[e] act(W1[e] x + b1[e]) + b2[e]  (SwiGLU: W2[e](silu(W1 x) * W3 x))
  y[t] = sum_j kept * g[t,j] * E_{i_j}(x_t)  (+ shared expert output)
  L_aux = E * sum_i f_i * P_i,  z = mean_t logsumexp(h_t)^2
and its backward pass: the gradients of <dy, y> + aux_coef L_aux + z_coef z with
respect to x, the router and every expert's weights (chain rule through each
step above; pinned by finite differences).

Readings of the pages (where they are silent or ambiguous) are marked READING
in the function that takes them. Every function here is pinned by a CPU test
against values the pages print, closed forms, brute force or library routines.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, Optional

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64
F32 = np.float32


# --------------------------------------------------------------------------
# Capacity
# --------------------------------------------------------------------------
def capacity(tokens: int, num_experts: int, top_k: int, capacity_factor: float,
             min_capacity: int, drop_tokens: bool) -> Optional[int]:
    """Per-expert capacity, or None when there is no limit.

    MoE Training Guide, "Core MoE Parameters" items 4-7: capacity is
    (tokens / num_experts) x capacity_factor, at least min_capacity, and
    disabling token dropping removes the limit.
    READING: "tokens" counts the T*k token-expert assignments (with T alone a
    top-2 layer at factor 1.25 would drop >= 37.5% under perfect balance, which
    the guide's "no dropping at 2.0" and "< 5% drop rate" contradict), and the
    quotient is rounded up. The factor is taken at its exact binary value.
    """
    if not drop_tokens:
        return None
    c = math.ceil(Fraction(capacity_factor) * (top_k * tokens) / num_experts)
    return max(int(min_capacity), int(c))


# --------------------------------------------------------------------------
# Router
# --------------------------------------------------------------------------
def router_logits(x, w_gate, b_gate=None) -> np.ndarray:
    """h(x) = x . W_g (+ b_g), W_g stored [E, d] as nn.Linear stores it.

    MoE From Scratch to DeepSeek V3, token-choice formula (score h(x) = x W_g);
    MoE Training: Mixture of Experts, "Basic MoE Architecture" (gate is an
    nn.Linear, with bias). Accumulated in float64, delivered as float32: the
    router's working precision.
    """
    h = np.asarray(x, F64) @ np.asarray(w_gate, F64).T
    if b_gate is not None:
        h = h + np.asarray(b_gate, F64)[None, :]
    return h.astype(F32)


def softmax_scores(logits) -> tuple:
    """p = softmax over the expert axis, and the per-token logsumexp.

    MoE From Scratch to DeepSeek V3, gating p = Softmax(h(x)); the survey's
    summaries normalise along the expert dimension. Returns (p, lse) in float64
    computed from the float32 logits.
    """
    h = np.asarray(logits, F64)
    m = h.max(axis=1, keepdims=True)
    e = np.exp(h - m)
    s = e.sum(axis=1, keepdims=True)
    return e / s, (m + np.log(s))[:, 0]


def logsumexp(logits) -> np.ndarray:
    """log(sum_e exp(h_e)) per token (router z-loss argument)."""
    return softmax_scores(logits)[1]


def sigmoid_scores(logits) -> np.ndarray:
    """s = 1 / (1 + exp(-h)) per expert (DeepSeek V3 sigmoid routing)."""
    h = np.asarray(logits, F64)
    return 1.0 / (1.0 + np.exp(-h))


def selection_keys(logits, score_fn: str, e_bias=None) -> np.ndarray:
    """The float32 value each token ranks experts by.

    softmax: top-k of p equals top-k of the logits because softmax is strictly
    increasing in each logit, so the key is the float32 logit itself (the
    Switch top-1 rule also selects on logits: MoE Training: Mixture of Experts,
    "2. Routing Mechanisms").
    sigmoid: key = s + b_i with the selection bias b_i (MoE From Scratch to
    DeepSeek V3, auxiliary-loss-free balancing, Score_i = x e_i + b_i).
    READING: the bias is added to the sigmoid score (not the raw logit) and the
    sum is formed in float32, the router's precision: s is the correctly rounded
    float32 sigmoid, then s + b in float32.
    """
    h = np.asarray(logits, F32)
    if score_fn == "softmax":
        return h.copy()
    if score_fn == "sigmoid":
        s32 = sigmoid_scores(h).astype(F32)
        b = np.zeros(h.shape[1], F32) if e_bias is None else np.asarray(e_bias, F32)
        return (s32 + b[None, :]).astype(F32)
    raise ValueError(score_fn)


def top_k(keys, k: int) -> np.ndarray:
    """Indices of the k largest keys per token, in descending key order.

    torch.topk in the pages' layers (MoE Training: Mixture of Experts, "Basic
    MoE Architecture"; moe_code.py, MixtureOfExperts.forward step 2).
    READING: equal keys go to the lower expert index first (torch.topk leaves
    this open). A stable sort of the negated keys gives exactly that order.
    """
    keys = np.asarray(keys)
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_margin(keys, k: int) -> np.ndarray:
    """key of the k-th choice minus key of the (k+1)-th (inf when k == E).

    Used by parity tests to set aside tokens whose selection is a near tie
    (the top-k decision taken on keys closer than a threshold may go either
    way). Pinned against a brute force over all k-subsets and hand cases.
    """
    keys = np.asarray(keys, F64)
    T, E = keys.shape
    if k >= E:
        return np.full(T, np.inf)
    srt = -np.sort(-keys, axis=1)
    return srt[:, k - 1] - srt[:, k]


def renormalised_gates(scores, idx) -> np.ndarray:
    """g_j = score_{i_j} / sum_{j'} score_{i_j'} over the k selected experts.

    moe_code.py, MixtureOfExperts.forward step 3, and MoE Training: Mixture of
    Experts, "Top-2 Routing (Mixtral)": divide the top-k scores by their sum.
    For the sigmoid router the scores are the unbiased sigmoid values (the
    selection bias only steers selection). k = 1 gives g = 1 (SwitchMoE).
    """
    sel = np.take_along_axis(np.asarray(scores, F64), np.asarray(idx, np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(logits, top_k_: int, score_fn: str, e_bias=None) -> Dict[str, np.ndarray]:
    """Score function, top-k and gates from float32 logits."""
    keys = selection_keys(logits, score_fn, e_bias)
    idx = top_k(keys, top_k_)
    if score_fn == "softmax":
        scores, lse = softmax_scores(logits)
    else:
        scores = sigmoid_scores(logits)
        lse = logsumexp(logits)
    gates = renormalised_gates(scores, idx)
    return dict(keys=keys, idx=idx, gates=gates, scores=scores, lse=lse,
                margin=topk_margin(keys, top_k_))


# --------------------------------------------------------------------------
# Dispatch (capacity, histogram, expert-sorted order)
# --------------------------------------------------------------------------
def dispatch(idx, num_experts: int, cap: Optional[int]) -> Dict[str, np.ndarray]:
    """Capacity-limited dispatch of the T*k assignments.

    MoE From Scratch to DeepSeek V3, "Token Dropping": once an expert's buffer
    is full the extra tokens are dropped. MoE Training Guide, "Core MoE
    Parameters" items 4-7 (capacity, min capacity, no-drop mode).
    READING: the queue order is k-major then token-ascending (every token's
    first choice before any second choice), so a higher-ranked choice never
    loses its slot to a lower-ranked one; a dropped assignment contributes
    nothing and the surviving gates are not renormalised again.

    Rows of the expert-sorted buffer are ordered by expert, then queue position.
    Returns counts_pre [E] (picks before capacity), counts_kept [E],
    expert_offsets [E+1], assign_row [T,k] (row or -1), row_token [R],
    row_slot [R] (the choice j of each row), pos [T,k], dropped.
    """
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    E = int(num_experts)
    flat = idx.T.reshape(-1)                       # a = j*T + t
    A = flat.size
    counts_pre = np.bincount(flat, minlength=E)[:E]
    order = np.argsort(flat, kind="stable")        # by expert, then queue order
    starts = np.cumsum(counts_pre) - counts_pre
    pos = np.empty(A, np.int64)
    pos[order] = np.arange(A) - starts[flat[order]]
    kept = np.ones(A, bool) if cap is None else pos < cap
    counts_kept = counts_pre.copy() if cap is None else np.minimum(counts_pre, cap)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts_kept)
    row = np.where(kept, offsets[flat] + pos, -1)
    R = int(offsets[-1])
    row_token = np.empty(R, np.int64)
    row_slot = np.empty(R, np.int64)
    a_kept = np.nonzero(kept)[0]
    row_token[row[a_kept]] = a_kept % T
    row_slot[row[a_kept]] = a_kept // T
    return dict(
        counts_pre=counts_pre.astype(np.int64),
        counts_kept=counts_kept.astype(np.int64),
        expert_offsets=offsets,
        assign_row=row.reshape(k, T).T.copy(),
        row_token=row_token,
        row_slot=row_slot,
        pos=pos.reshape(k, T).T.copy(),
        dropped=int(A - R),
    )


# --------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------
def gelu(z):
    """Exact GELU, 0.5 z (1 + erf(z / sqrt 2)): nn.GELU() default, used by the
    expert FFN in MoE Training: Mixture of Experts, "Basic MoE Architecture"."""
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def relu(z):
    """max(z, 0): moe_code.py, class Expert."""
    return np.maximum(z, 0.0)


def silu(z):
    """z / (1 + exp(-z)), the gate nonlinearity of SwiGLU."""
    return z / (1.0 + np.exp(-z))


def expert_ffn(xr, w1, b1, w2, b2, activation: str, w3=None) -> np.ndarray:
    """One expert on rows xr [n, d]: W2 act(W1 x + b1) + b2, weights [out, in].

    GELU/ReLU: MoE Training: Mixture of Experts, "Basic MoE Architecture"
    (Linear(h, 4h), GELU, Linear(4h, h)) and moe_code.py, class Expert
    (ReLU(x W1 + b1) W2 + b2; its dropout is the identity in a forward
    evaluation).
    SwiGLU: three matrices per expert (Moe survey, Mixtral parameter count).
    READING: H = silu(W1 x) * (W3 x), output W2 H.
    """
    xr = np.asarray(xr, F64)
    W1 = np.asarray(w1, F64)
    h = xr @ W1.T
    if b1 is not None:
        h = h + np.asarray(b1, F64)[None, :]
    if activation == "gelu":
        h = gelu(h)
    elif activation == "relu":
        h = relu(h)
    elif activation == "swiglu":
        u = xr @ np.asarray(w3, F64).T
        h = silu(h) * u
    else:
        raise ValueError(activation)
    y = h @ np.asarray(w2, F64).T
    if b2 is not None:
        y = y + np.asarray(b2, F64)[None, :]
    return y


def experts_forward(x, disp: Dict[str, np.ndarray], params, activation: str) -> np.ndarray:
    """Y[r] = E_e(x[row_token[r]]) for every kept row r of expert e."""
    x = np.asarray(x, F64)
    offsets = disp["expert_offsets"]
    R = int(offsets[-1])
    Y = np.zeros((R, x.shape[1]), F64)
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = x[disp["row_token"][lo:hi]]
        Y[lo:hi] = expert_ffn(rows, params["w1"][e], _opt(params.get("b1"), e),
                              params["w2"][e], _opt(params.get("b2"), e), activation,
                              _opt(params.get("w3"), e))
    return Y


def _opt(t, e):
    return None if t is None else t[e]


def combine(Y, gates, assign_row, T: int, d: int, y_shared=None) -> np.ndarray:
    """y[t] = sum_j kept * g[t, j] * Y[assign_row[t, j]] (+ y_shared[t]).

    MoE From Scratch to DeepSeek V3, output y = sum over TopK of Gate_i E_i(x);
    MoE Training: Mixture of Experts, "Weighted Combination".
    READING: the layer returns the mixture without the "+ x" residual of the
    lecture's formula (the page's own layer code adds none; the residual belongs
    to the transformer block). Shared experts are always active with gate 1
    (MoE From Scratch to DeepSeek V3, "Shared Experts").
    """
    y = np.zeros((T, d), F64)
    k = assign_row.shape[1]
    for j in range(k):
        r = assign_row[:, j]
        ok = r >= 0
        y[ok] += np.asarray(gates, F64)[ok, j:j + 1] * Y[r[ok]]
    if y_shared is not None:
        y += y_shared
    return y


# --------------------------------------------------------------------------
# Balance statistics
# --------------------------------------------------------------------------
def balance_stats(scores, score_fn: str, lse, counts_pre, counts_kept, T: int, k: int,
                  E: int) -> Dict[str, float]:
    """f_i, P_i, L_aux = E sum f_i P_i, z-loss and the monitoring figures.

    MoE Training: Mixture of Experts, "3. Load Balancing": f = bincount of the
    top-k indices / their number, P = mean softmax probability, aux = E sum f P;
    router z-loss = mean of logsumexp(logits)^2 (also MoE From Scratch to
    DeepSeek V3, L_aux = N sum f_i P_i and L_z = log^2 sum e^logit).
    MoE Training Guide, "Monitoring": load imbalance max/min counts, utilisation
    (experts with a nonzero count / E), drop rate (dropped / total).
    READING: f_i counts top-k picks before capacity (so sum f = 1 and uniform
    routing gives L_aux = 1); for the sigmoid router P_i is the mean of the
    per-token normalised affinities s_ti / sum_e s_te.
    """
    scores = np.asarray(scores, F64)
    if score_fn == "sigmoid":
        scores = scores / scores.sum(axis=1, keepdims=True)
    counts_pre = np.asarray(counts_pre, np.int64)
    counts_kept = np.asarray(counts_kept, np.int64)
    A = T * k
    f = counts_pre / float(A)
    P = scores.mean(axis=0)
    lse = np.asarray(lse, F64)
    kept = int(counts_kept.sum())
    cmin = int(counts_pre.min())
    return dict(
        f=f, P=P, l_aux=float(E * np.sum(f * P)), z_loss=float(np.mean(lse * lse)),
        kept=kept, dropped=A - kept, drop_rate=(A - kept) / float(A),
        utilization=float(np.count_nonzero(counts_kept > 0)) / E,
        imbalance=(float(counts_pre.max()) / cmin) if cmin > 0 else math.inf,
    )


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def forward(x, params, w, logits=None, idx=None) -> Dict[str, object]:
    """The full layer forward for workload ``w`` (a workloads.Workload-like object).

    ``params`` maps w_gate, b_gate, e_bias, w1, w3, b1, w2, b2 and the shared
    expert's ws1, ws3, bs1, ws2, bs2 to arrays indexable per expert. ``logits``
    (float32 [T, E]) may be given to run routing on another implementation's
    router output; ``idx`` likewise overrides the top-k choice (stage-isolated
    comparison). Returns every intermediate.
    """
    x = np.asarray(x, F64)
    T, d = x.shape
    E, k = w.num_experts, w.top_k
    if logits is None:
        logits = router_logits(x, params["w_gate"], params.get("b_gate"))
    r = route(logits, k, w.score_fn, params.get("e_bias"))
    if idx is not None:
        idx = np.asarray(idx, np.int32)
        r["idx"] = idx
        r["gates"] = renormalised_gates(r["scores"], idx)
    cap = capacity(T, E, k, w.capacity_factor, w.min_capacity, w.drop_tokens)
    disp = dispatch(r["idx"], E, cap)
    Y = experts_forward(x, disp, params, w.activation)
    y_shared = None
    if w.num_shared_experts:
        y_shared = np.zeros((T, d), F64)
        for s in range(w.num_shared_experts):
            y_shared += expert_ffn(x, params["ws1"][s], _opt(params.get("bs1"), s),
                                   params["ws2"][s], _opt(params.get("bs2"), s),
                                   w.activation, _opt(params.get("ws3"), s))
    y = combine(Y, r["gates"], disp["assign_row"], T, d, y_shared)
    stats = balance_stats(r["scores"], w.score_fn, r["lse"], disp["counts_pre"],
                          disp["counts_kept"], T, k, E)
    return dict(logits=np.asarray(logits, F32), capacity=cap, y=y, Y=Y, y_shared=y_shared,
                stats=stats, **r, **disp)


# --------------------------------------------------------------------------
# Parameter and FLOP accounting
# --------------------------------------------------------------------------
def ffn_params(d_model: int, d_ff: int, activation: str, bias: bool) -> int:
    """Parameters of one expert: two d x d_ff matrices (three for SwiGLU).

    moe_code.py, compare_moe_vs_dense (expert = 2 d d_ff, no biases counted);
    Moe survey, Mixtral count (three matrices per expert).
    """
    mats = 3 if activation == "swiglu" else 2
    n = mats * d_model * d_ff
    if bias:
        n += (mats - 1) * d_ff + d_model
    return n


def router_params(d_model: int, num_experts: int, bias: bool) -> int:
    """Gate parameters: d x E (+ E with a bias)."""
    return d_model * num_experts + (num_experts if bias else 0)


def layer_params(d_model, d_ff, num_experts, top_k, activation, bias=False, gate_bias=False,
                 num_shared=0) -> Dict[str, int]:
    """Total and active (per token) parameters of one MoE layer."""
    fe = ffn_params(d_model, d_ff, activation, bias)
    rg = router_params(d_model, num_experts, gate_bias)
    return dict(expert=fe, router=rg,
                total=(num_experts + num_shared) * fe + rg,
                active=(top_k + num_shared) * fe + rg)


def expert_flops(rows: int, d_model: int, d_ff: int, activation: str) -> int:
    """Multiply-add FLOPs (2 per MAC) of the expert matrices over ``rows`` rows."""
    mats = 3 if activation == "swiglu" else 2
    return 2 * rows * d_model * d_ff * mats


# --------------------------------------------------------------------------
# Backward pass (gradients of the layer)
# --------------------------------------------------------------------------
# The layer is differentiated through every path the forward above defines,
# with the scalar objective
#   L = <dy, y> + aux_coef * L_aux + z_coef * z
# i.e. dy is the gradient of the caller's loss with respect to the layer output
# and aux_coef / z_coef are the weights the loss puts on the balance loss and
# the router z-loss (MoE Training: Mixture of Experts, "3. Load Balancing":
# the auxiliary loss is added to the task loss with a small coefficient; MoE
# From Scratch to DeepSeek V3, router z-loss as a training loss).
# READING: the top-k choice, the capacity decision and the counts f_i are
# piecewise constant in the parameters and carry no gradient (the pages train
# the router only through the gate values, the probabilities P_i and the
# logsumexp); the sigmoid selection bias e_bias receives none either (it is
# moved by the balancing rule, not by the gradient).

def gelu_grad(z):
    """d/dz of exact GELU z Phi(z): Phi(z) + z phi(z)."""
    z = np.asarray(z, F64)
    return 0.5 * (1.0 + _erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def relu_grad(z):
    """d/dz max(z, 0): 1 for z > 0, else 0 (0 at the kink, as autograd takes it)."""
    return (np.asarray(z, F64) > 0.0).astype(F64)


def silu_grad(z):
    """d/dz z sigma(z) = sigma(z) (1 + z (1 - sigma(z)))."""
    z = np.asarray(z, F64)
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_ffn_backward(xr, w1, b1, w2, b2, activation: str, dY, w3=None) -> Dict[str, np.ndarray]:
    """Gradients of one expert E(x) = W2 act(W1 x + b1) + b2 on rows xr [n, d].

    Chain rule through expert_ffn (MoE Training: Mixture of Experts, "Basic MoE
    Architecture"; moe_code.py, class Expert; SwiGLU reading as in expert_ffn):
      dH = dY W2,  dW2 = dY^T H,  db2 = sum_rows dY
      dZ = dH * act'(Z)   (SwiGLU: dZ = dH * U * silu'(Z), dU = dH * silu(Z))
      dX = dZ W1 (+ dU W3),  dW1 = dZ^T X,  db1 = sum_rows dZ  (dW3 = dU^T X)
    Returns dx, dw1, db1, dw2, db2, dw3 (None where absent) and the
    intermediates z, u (SwiGLU), h, dz.
    """
    X = np.asarray(xr, F64)
    W1 = np.asarray(w1, F64)
    W2 = np.asarray(w2, F64)
    dY = np.asarray(dY, F64)
    Z = X @ W1.T
    if b1 is not None:
        Z = Z + np.asarray(b1, F64)[None, :]
    U = None
    if activation == "gelu":
        H = gelu(Z)
    elif activation == "relu":
        H = relu(Z)
    elif activation == "swiglu":
        U = X @ np.asarray(w3, F64).T
        H = silu(Z) * U
    else:
        raise ValueError(activation)
    dH = dY @ W2
    dW2 = dY.T @ H
    db2 = dY.sum(axis=0) if b2 is not None else None
    dW3 = None
    if activation == "gelu":
        dZ = dH * gelu_grad(Z)
    elif activation == "relu":
        dZ = dH * relu_grad(Z)
    else:
        dZ = dH * U * silu_grad(Z)
        dU = dH * silu(Z)
        dW3 = dU.T @ X
    dX = dZ @ W1
    if activation == "swiglu":
        dX = dX + dU @ np.asarray(w3, F64)
    dW1 = dZ.T @ X
    db1 = dZ.sum(axis=0) if b1 is not None else None
    return dict(dx=dX, dw1=dW1, db1=db1, dw2=dW2, db2=db2, dw3=dW3, z=Z, u=U, h=H, dz=dZ)


def combine_backward(dy, Y, gates, assign_row) -> tuple:
    """Gradients of combine: dY[r] = g[t,j] dy[t] and dg[t,j] = <dy[t], Y[r]>
    for the kept assignments (r = assign_row[t,j] >= 0); dropped ones get 0.

    MoE From Scratch to DeepSeek V3, y = sum_{TopK} Gate_i E_i(x); MoE Training:
    Mixture of Experts, "Weighted Combination". The shared expert's rows receive
    dy itself (gate 1); that part is handled by the caller.
    """
    dy = np.asarray(dy, F64)
    Y = np.asarray(Y, F64)
    gates = np.asarray(gates, F64)
    T, k = assign_row.shape
    dY = np.zeros_like(Y)
    dg = np.zeros((T, k), F64)
    for j in range(k):
        r = assign_row[:, j]
        ok = r >= 0
        dY[r[ok]] = gates[ok, j:j + 1] * dy[ok]
        dg[ok, j] = np.einsum("td,td->t", dy[ok], Y[r[ok]])
    return dY, dg


def router_backward(logits, idx, score_fn: str, dgate, f, aux_coef: float, z_coef: float) -> np.ndarray:
    """Gradient of the objective with respect to the router logits h [T, E].

    Three terms, each the derivative of a forward definition:
    1. Gates g_j = s_{i_j} / S, S = sum of the k selected scores (renormalised_gates):
       dS-rule gives ds_{i_m} = (dg_m - sum_j dg_j g_j) / S for the selected experts.
    2. L_aux = E sum_i f_i P_i with P_i = mean_t q_ti (balance_stats): q = p for the
       softmax router, q = s / sum_e s for the sigmoid router; f is constant, so
       dL_aux/dq_ti = E f_i / T. For the sigmoid router this is taken back through the
       normalisation: ds_ti += (dq_ti - sum_e dq_te q_te) / sum_e s_te.
    3. Scores to logits: softmax Jacobian dh = p * (dp - sum_e dp_e p_e), or sigmoid
       dh = ds * s (1 - s). Router z-loss z = mean_t lse_t^2 (MoE From Scratch to
       DeepSeek V3, router z-loss) adds 2 lse_t softmax(h_t) / T whatever the score
       function.
    """
    h = np.asarray(logits, F64)
    T, E = h.shape
    idx = np.asarray(idx, np.int64)
    dgate = np.asarray(dgate, F64)
    f = np.asarray(f, F64)
    p, lse = softmax_scores(h)
    s = p if score_fn == "softmax" else sigmoid_scores(h)
    sel = np.take_along_axis(s, idx, axis=1)
    S = sel.sum(axis=1, keepdims=True)
    g = sel / S
    dsel = (dgate - (dgate * g).sum(axis=1, keepdims=True)) / S
    ds = np.zeros((T, E), F64)
    np.put_along_axis(ds, idx, dsel, axis=1)   # the k selected experts are distinct
    dq = np.broadcast_to(aux_coef * E * f[None, :] / T, (T, E))
    if score_fn == "softmax":
        ds = ds + dq
        dh = p * (ds - (ds * p).sum(axis=1, keepdims=True))
    else:
        tot = s.sum(axis=1, keepdims=True)
        q = s / tot
        ds = ds + (dq - (dq * q).sum(axis=1, keepdims=True)) / tot
        dh = ds * s * (1.0 - s)
    dh = dh + z_coef * 2.0 * lse[:, None] * p / T
    return dh


def backward(x, params, w, dy, aux_coef: float = 0.0, z_coef: float = 0.0, fwd=None,
             logits=None) -> Dict[str, object]:
    """All gradients of the layer for workload ``w``.

    ``fwd`` is the result of forward() for the same inputs (computed here when
    None); passing one computed with another implementation's routing choice
    gives the stage-isolated comparison; ``logits`` overrides the logits the
    router gradient is taken at (default: the float32 logits of ``fwd``). Returns dx, dw_gate, db_gate, dw1, db1,
    dw2, db2, dw3, the shared expert's dws1, dbs1, dws2, dbs2, dws3, and the
    intermediates dY (expert-sorted rows), dgate, dlogits, z (pre-activation per
    row) and dz.
    """
    x = np.asarray(x, F64)
    T, d = x.shape
    E, k = w.num_experts, w.top_k
    if fwd is None:
        fwd = forward(x, params, w)
    act = w.activation
    dy = np.asarray(dy, F64)
    offsets = fwd["expert_offsets"]
    R = int(offsets[-1])
    dY, dgate = combine_backward(dy, fwd["Y"], fwd["gates"], fwd["assign_row"])
    F = np.asarray(params["w1"][0]).shape[0]
    dx = np.zeros((T, d), F64)
    out = dict(dw1=np.zeros((E, F, d), F64), dw2=np.zeros((E, d, F), F64),
               db1=np.zeros((E, F), F64) if params.get("b1") is not None else None,
               db2=np.zeros((E, d), F64) if params.get("b2") is not None else None,
               dw3=np.zeros((E, F, d), F64) if act == "swiglu" else None)
    Z = np.zeros((R, F), F64)
    U = np.zeros((R, F), F64) if act == "swiglu" else None
    dZ = np.zeros((R, F), F64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = fwd["row_token"][lo:hi]
        gr = expert_ffn_backward(x[toks], params["w1"][e], _opt(params.get("b1"), e),
                                 params["w2"][e], _opt(params.get("b2"), e), act, dY[lo:hi],
                                 _opt(params.get("w3"), e))
        np.add.at(dx, toks, gr["dx"])
        out["dw1"][e] = gr["dw1"]
        out["dw2"][e] = gr["dw2"]
        if out["db1"] is not None:
            out["db1"][e] = gr["db1"]
            out["db2"][e] = gr["db2"]
        if act == "swiglu":
            out["dw3"][e] = gr["dw3"]
        Z[lo:hi] = gr["z"]
        if U is not None:
            U[lo:hi] = gr["u"]
        dZ[lo:hi] = gr["dz"]
    if w.num_shared_experts:
        gs = expert_ffn_backward(x, params["ws1"][0], _opt(params.get("bs1"), 0), params["ws2"][0],
                                 _opt(params.get("bs2"), 0), act, dy, _opt(params.get("ws3"), 0))
        dx += gs["dx"]
        out.update(dws1=gs["dw1"], dbs1=gs["db1"], dws2=gs["dw2"], dbs2=gs["db2"], dws3=gs["dw3"],
                   z_shared=gs["z"], u_shared=gs["u"], dz_shared=gs["dz"])
    f = np.asarray(fwd["counts_pre"], F64) / float(T * k)
    dlogits = router_backward(fwd["logits"] if logits is None else logits, fwd["idx"],
                              w.score_fn, dgate, f, aux_coef, z_coef)
    Wg = np.asarray(params["w_gate"], F64)
    dx += dlogits @ Wg
    out.update(dx=dx, dw_gate=dlogits.T @ x,
               db_gate=dlogits.sum(axis=0) if params.get("b_gate") is not None else None,
               dY=dY, dgate=dgate, dlogits=dlogits, z=Z, u=U, dz=dZ)
    return out


# --------------------------------------------------------------------------
# Expert-choice routing
# --------------------------------------------------------------------------
# Each expert picks its C best tokens over the transposed [E, T] scores, so every
# expert is exactly full (MoE Training: Mixture of Experts, "2. Routing
# Mechanisms", expert choice routing: experts choose top-k tokens, which
# guarantees perfect load balancing; MoE From Scratch to DeepSeek V3: expert
# choice keeps the load balanced but may treat tokens unevenly; the survey's
# expert-choice routing entry).
# READINGS: the score an expert ranks tokens by is the router logit (the page's
# router(x) is the logit, as in its top-1 code), in float32; equal scores go to
# the lower token index first; the weight of an expert's output for a token is
# the router score: the softmax probability p[t, e] over experts (the
# token-choice gate p = Softmax(h(x)) of MoE From Scratch to DeepSeek V3), or for
# the sigmoid router the sigmoid score s[t, e] (there is no top-k set to
# renormalise over); a token no expert picks gets zero (plus the shared expert);
# C is the capacity rule of capacity() with k the average experts per token,
# ceil(k T / E) when dropping is off, and never more than T; an expert's rows are
# its chosen tokens in ascending token order.

def expert_choice_capacity(tokens: int, num_experts: int, top_k: int, capacity_factor: float,
                           min_capacity: int, drop_tokens: bool) -> int:
    """Tokens per expert C for expert-choice routing (see the readings above)."""
    c = capacity(tokens, num_experts, top_k, capacity_factor, min_capacity, drop_tokens)
    if c is None:
        c = -(-top_k * tokens // num_experts)
    return int(min(c, tokens))


def expert_choice_route(logits, C: int, score_fn: str = "softmax") -> Dict[str, np.ndarray]:
    """Per expert, the C tokens with the largest float32 logit (ties: lower token
    first), listed in ascending token order; their gates; the row of (t, e) or -1.

    Gates: softmax router, p[t, e] (softmax over experts); sigmoid router, the
    sigmoid score s[t, e] itself. READING: the pages weight an expert's output
    by the router's score for (t, e) and give no renormalisation for expert
    choice (a token has no fixed number of picks), so the sigmoid gate is the
    raw score. Both scores increase with the logit, so an expert's C best tokens
    by score are its C best by logit; the logit is the key (float32 rounding of
    the score could make distinct logits equal). affinity: the per-token
    distribution over experts that P_i averages (p, or s / sum_e s as in the
    token-choice statistics).

    Rows: expert e's chosen tokens occupy rows e C .. e C + C - 1.
    """
    h32 = np.asarray(logits, F32)
    T, E = h32.shape
    if score_fn == "softmax":
        scores, lse = softmax_scores(h32)
        affinity = scores
    elif score_fn == "sigmoid":
        scores = sigmoid_scores(h32)
        lse = logsumexp(h32)
        affinity = scores / scores.sum(axis=1, keepdims=True)
    else:
        raise ValueError(score_fn)
    tokens = np.empty((E, C), np.int64)
    for e in range(E):
        order = np.argsort(-h32[:, e], kind="stable")   # descending, lower token first on ties
        tokens[e] = np.sort(order[:C])
    gates = np.take_along_axis(scores.T, tokens, axis=1)  # [E, C]
    row = np.full((T, E), -1, np.int64)
    for e in range(E):
        row[tokens[e], e] = e * C + np.arange(C)
    picks = (row >= 0).sum(axis=1)
    return dict(tokens=tokens, gates=gates, row=row, scores=scores, affinity=affinity, lse=lse,
                picks=picks)


def expert_choice_forward(x, params, w, logits=None) -> Dict[str, object]:
    """The layer with expert-choice routing: y[t] = sum over the experts e that
    picked t of gate[t, e] E_e(x_t) (+ shared expert). Statistics: every expert
    takes C tokens; "unpicked" counts the tokens no expert chose; P_i (mean
    affinity) and the z-loss as for token choice."""
    x = np.asarray(x, F64)
    T, d = x.shape
    E = w.num_experts
    C = expert_choice_capacity(T, E, w.top_k, w.capacity_factor, w.min_capacity, w.drop_tokens)
    if logits is None:
        logits = router_logits(x, params["w_gate"], params.get("b_gate"))
    r = expert_choice_route(logits, C, w.score_fn)
    Y = np.zeros((E * C, d), F64)
    for e in range(E):
        Y[e * C:(e + 1) * C] = expert_ffn(x[r["tokens"][e]], params["w1"][e], _opt(params.get("b1"), e),
                                          params["w2"][e], _opt(params.get("b2"), e), w.activation,
                                          _opt(params.get("w3"), e))
    y = np.zeros((T, d), F64)
    for e in range(E):
        y[r["tokens"][e]] += r["gates"][e][:, None] * Y[e * C:(e + 1) * C]
    if w.num_shared_experts:
        y += expert_ffn(x, params["ws1"][0], _opt(params.get("bs1"), 0), params["ws2"][0],
                        _opt(params.get("bs2"), 0), w.activation, _opt(params.get("ws3"), 0))
    stats = dict(capacity=C, P=r["affinity"].mean(axis=0), z_loss=float(np.mean(r["lse"] ** 2)),
                 unpicked=int(np.count_nonzero(r["picks"] == 0)), max_picks=int(r["picks"].max()))
    return dict(logits=np.asarray(logits, F32), y=y, Y=Y, stats=stats, C=C, **r)


# --------------------------------------------------------------------------
# Auxiliary-loss-free balancing: the selection-bias update
# --------------------------------------------------------------------------
def update_selection_bias(e_bias, counts_pre, tokens: int, top_k: int, gamma: float) -> np.ndarray:
    """One update of the sigmoid router's selection bias b_i.

    MoE From Scratch to DeepSeek V3, auxiliary-loss-free balancing: b_i is lowered
    when expert i is overloaded and raised when it is idle.
    READING: "overloaded" / "idle" compare the expert's top-k picks (before
    capacity) with the mean load T k / E, exactly (in integers: c_i E against
    T k); the step is a caller-given gamma (the pages give none), b_i <- b_i -
    gamma sign(c_i - T k / E), evaluated in float32 (the bias is a float32
    router quantity).
    """
    b = np.asarray(e_bias, F32).copy()
    c = np.asarray(counts_pre, np.int64)
    E = b.shape[0]
    s = np.sign(c * E - tokens * top_k)            # exact: +1 over, -1 under, 0 at the mean
    return (b - F32(gamma) * s.astype(F32)).astype(F32)


# --------------------------------------------------------------------------
# Hash routing
# --------------------------------------------------------------------------
def hash_route(token_ids, table) -> np.ndarray:
    """Expert of each token from a fixed token-id -> expert map.

    Moe(Mixtrue of Experts) survey: hash-based routing fixes the token -> expert
    mapping in advance (no gating network), which removes the fluctuation of a
    learned router; its "Hash layers for large sparse models" entry routes each
    token by hashing it.
    READING: the map is a table indexed by token id, given by the caller (how it
    is generated is the caller's choice); one expert per token (k = 1) with gate
    1. Ids outside [0, V) and table entries outside [0, E) are clamped (the
    library has to stay memory-safe on any input).
    """
    ids = np.clip(np.asarray(token_ids, np.int64), 0, len(table) - 1)
    return np.asarray(table, np.int64)[ids].reshape(-1, 1)


def hash_forward(x, params, w, token_ids, table) -> Dict[str, object]:
    """The layer with hash routing: idx = table[token id] (k = 1, gate 1), then
    the capacity-limited dispatch, the experts and the combine of the token-choice
    layer (plus the shared expert). No router: P_i and the z-loss are 0."""
    x = np.asarray(x, F64)
    T, d = x.shape
    E = w.num_experts
    idx = np.clip(hash_route(token_ids, table), 0, E - 1)
    gates = np.ones((T, 1), F64)
    cap = capacity(T, E, 1, w.capacity_factor, w.min_capacity, w.drop_tokens)
    disp = dispatch(idx, E, cap)
    Y = experts_forward(x, disp, params, w.activation)
    y_shared = None
    if w.num_shared_experts:
        y_shared = expert_ffn(x, params["ws1"][0], _opt(params.get("bs1"), 0), params["ws2"][0],
                              _opt(params.get("bs2"), 0), w.activation, _opt(params.get("ws3"), 0))
    y = combine(Y, gates, disp["assign_row"], T, d, y_shared)
    return dict(idx=idx.astype(np.int32), gates=gates, y=y, Y=Y, capacity=cap, **disp)
