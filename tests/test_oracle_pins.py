"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print, closed forms, brute-force enumeration, literal simulations of the
definition, or library routines (torch CPU float64) for special cases.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn
from scipy.special import softmax as sp_softmax

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- accounting
def test_mixtral_parameter_count_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "mixtral_8x7b_params.json")))
    lp = O.layer_params(g["d_model"], g["d_ff"], g["num_experts"], g["top_k"], "swiglu",
                        bias=False, gate_bias=False)
    assert lp["expert"] == g["expert_ffn_params"]
    L = g["layers"]
    assert lp["expert"] * g["num_experts"] * L == g["all_layers_expert_ffn_params"]
    assert lp["router"] * L == g["all_layers_gate_params"]
    per_layer = lp["total"] + g["attention_params_per_layer"] + g["layernorm_params_per_layer"]
    assert per_layer * L == g["transformer_total"]
    assert per_layer * L + g["embed_and_output_params"] == g["total"]
    active_layer = lp["active"] + g["attention_params_per_layer"] + g["layernorm_params_per_layer"]
    assert active_layer * L + g["embed_and_output_params"] == g["active"]


def test_moe_vs_dense_accounting_closed_forms():
    # moe_code.py, compare_moe_vs_dense at its default (768, 3072, 8, 2):
    # dense 2*d*dff, MoE total E*2*d*dff + d*E, active k*2*d*dff + d*E.
    lp = O.layer_params(768, 3072, 8, 2, "gelu", bias=False, gate_bias=False)
    assert lp["expert"] == 4_718_592
    assert lp["total"] == 37_754_880
    assert lp["active"] == 9_443_328
    # biases of nn.Linear(d, F) and nn.Linear(F, d)
    assert O.ffn_params(32, 128, "gelu", True) == 2 * 32 * 128 + 128 + 32
    assert O.router_params(32, 4, True) == 32 * 4 + 4
    assert O.expert_flops(10, 768, 3072, "gelu") == 10 * 2 * (2 * 768 * 3072)


# ---------------------------------------------------------------- capacity
def test_capacity_values():
    # DeepSpeed GPT-MoE shape: T=8192, E=8, k=2, factor 1.25 -> 2560 slots per expert
    assert O.capacity(8192, 8, 2, 1.25, 4, True) == 2560
    # 128 experts, top-1: train factor 1.25 -> 80, eval factor 2.0 -> 128
    assert O.capacity(8192, 128, 1, 1.25, 4, True) == 80
    assert O.capacity(8192, 128, 1, 2.0, 4, True) == 128
    # min_capacity binds: ceil(1 * 8 / 8) = 1 < 4
    assert O.capacity(8, 8, 1, 1.0, 4, True) == 4
    # dropping disabled: no limit
    assert O.capacity(8192, 8, 2, 1.25, 4, False) is None
    # rounding up of a non-integer quotient: 1.25 * 2 * 100 / 8 = 31.25 -> 32
    assert O.capacity(100, 8, 2, 1.25, 4, True) == 32


def test_capacity_uses_exact_factor_value():
    # The double nearest 0.3 is slightly below 0.3, so 10 * it is just below 3.
    from decimal import Decimal
    assert Decimal(0.3) * 10 < 3
    assert O.capacity(10, 1, 1, 0.3, 0, True) == 3
    # and the double nearest 1.1 is above 1.1: 10 * it is just above 11
    assert Decimal(1.1) * 10 > 11
    assert O.capacity(10, 1, 1, 1.1, 0, True) == 12


# ---------------------------------------------------------------- top-k
def _brute_topk(keys_row, k):
    E = len(keys_row)
    best, best_sum = None, None
    for S in itertools.combinations(range(E), k):      # lexicographic order
        s = sum(float(keys_row[i]) for i in S)
        if best_sum is None or s > best_sum:
            best, best_sum = S, s
    return sorted(best, key=lambda i: (-float(keys_row[i]), i))


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (6, 3), (8, 2), (8, 8), (5, 4)])
def test_topk_matches_subset_enumeration(E, k):
    rng = np.random.default_rng(E * 10 + k)
    keys = rng.integers(0, 4, size=(200, E)).astype(np.float32)   # many exact ties
    idx = O.top_k(keys, k)
    for t in range(keys.shape[0]):
        assert list(idx[t]) == _brute_topk(keys[t], k), (t, keys[t])


def test_topk_on_logits_equals_topk_on_probabilities():
    rng = np.random.default_rng(1)
    logits = rng.normal(size=(300, 16)).astype(np.float32)
    p, _ = O.softmax_scores(logits)
    r = O.route(logits, 3, "softmax")
    ref = torch.topk(torch.from_numpy(p), 3, dim=-1).indices.numpy()
    assert np.array_equal(r["idx"], ref)


def test_top2_worked_example_gates():
    g = json.load(open(os.path.join(GOLDEN, "top2_worked_example.json")))
    logits = np.asarray([g["logits"]], np.float32)
    r = O.route(logits, g["top_k"], "softmax")
    assert list(r["idx"][0]) == g["expected_idx"]
    assert np.allclose(r["gates"][0], g["expected_gates"], rtol=0, atol=1e-6)


# ---------------------------------------------------------------- gates
def test_gates_sum_to_one_and_match_restricted_softmax():
    rng = np.random.default_rng(2)
    logits = rng.normal(scale=2.0, size=(128, 8)).astype(np.float32)
    for k in (1, 2, 4):
        r = O.route(logits, k, "softmax")
        assert np.allclose(r["gates"].sum(1), 1.0, rtol=0, atol=1e-15)
        sel = np.take_along_axis(logits.astype(np.float64), r["idx"].astype(np.int64), 1)
        assert np.allclose(r["gates"], sp_softmax(sel, axis=1), rtol=1e-13, atol=0)
        if k == 1:
            assert np.all(r["gates"] == 1.0)


def test_sigmoid_bias_steers_selection_not_gates():
    logits = np.array([[0.0, 0.1, -0.1]], np.float32)
    e_bias = np.array([0.0, 0.0, 0.5], np.float32)
    r1 = O.route(logits, 1, "sigmoid", e_bias)
    assert list(r1["idx"][0]) == [2] and r1["gates"][0, 0] == 1.0
    r2 = O.route(logits, 2, "sigmoid", e_bias)
    assert list(r2["idx"][0]) == [2, 1]
    # sigma(x) + sigma(-x) = 1, so the renormalised unbiased gates are sigma(-0.1), sigma(0.1)
    h = float(np.float32(0.1))
    assert np.allclose(r2["gates"][0], [1 / (1 + math.exp(h)), 1 / (1 + math.exp(-h))],
                       rtol=1e-12, atol=0)
    # without bias the same logits pick expert 1 first
    r3 = O.route(logits, 1, "sigmoid", None)
    assert list(r3["idx"][0]) == [1]


def test_sigmoid_scores_match_torch():
    rng = np.random.default_rng(3)
    l = rng.normal(scale=3, size=(50, 9)).astype(np.float32)
    assert np.allclose(O.sigmoid_scores(l), torch.sigmoid(torch.from_numpy(l).double()).numpy(),
                       rtol=1e-14, atol=0)



# ---------------------------------------------------------------- top-k margin
def _margin_by_subsets(keys, k):
    """The selection's margin as a brute force over every k-subset S of the
    experts: the largest value of min(keys in S) - max(keys outside S). The
    top-k set attains key_(k) - key_(k+1) >= 0; every other set scores <= 0;
    with k = E there is nothing outside S (margin +inf)."""
    E = len(keys)
    if k >= E:
        return math.inf
    best = -math.inf
    for S in itertools.combinations(range(E), k):
        inside = min(keys[i] for i in S)
        outside = max(keys[i] for i in range(E) if i not in S)
        best = max(best, inside - outside)
    return best


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (7, 6), (8, 4)])
def test_topk_margin_matches_subset_brute_force(E, k):
    rng = np.random.default_rng(100 + E * 10 + k)
    # integer keys with many ties, plus continuous keys
    keys = np.concatenate([rng.integers(-3, 4, size=(30, E)).astype(np.float32),
                           rng.normal(size=(30, E)).astype(np.float32)])
    m = O.topk_margin(keys, k)
    ref = np.array([_margin_by_subsets([float(v) for v in row], k) for row in keys])
    assert np.array_equal(m, ref)
    assert np.all(m >= 0)


def test_topk_margin_hand_cases():
    # keys 0.5, 0.9, 0.1, 0.7: top-2 = {0.9, 0.7}, the next key is 0.5
    keys = np.array([[0.5, 0.9, 0.1, 0.7]], np.float64)
    assert O.topk_margin(keys, 2)[0] == pytest.approx(0.2, abs=1e-15)
    assert O.topk_margin(keys, 1)[0] == pytest.approx(0.2, abs=1e-15)   # 0.9 - 0.7
    assert O.topk_margin(keys, 3)[0] == pytest.approx(0.4, abs=1e-15)   # 0.5 - 0.1
    # k = E: no competitor, the choice cannot flip
    assert O.topk_margin(keys, 4)[0] == math.inf
    # an exact tie at the boundary gives 0 (either expert is a correct choice)
    tie = np.array([[1.0, 3.0, 1.0, -2.0]], np.float32)
    assert O.topk_margin(tie, 2)[0] == 0.0
    assert O.topk_margin(tie, 1)[0] == 2.0
    # the margin is on the keys the routing ranks by (sigmoid: s + bias)
    l = np.array([[0.0, 0.0]], np.float32)
    keys_s = O.selection_keys(l, "sigmoid", np.array([0.25, 0.0], np.float32))
    assert O.topk_margin(keys_s, 1)[0] == 0.25

# ---------------------------------------------------------------- statistics
@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (16, 4)])
def test_laux_is_one_under_uniform_routing(E, k):
    v = np.linspace(1.0, -1.0, E).astype(np.float32)         # distinct entries
    T = 3 * E
    logits = np.stack([np.roll(v, t) for t in range(T)])
    r = O.route(logits, k, "softmax")
    d = O.dispatch(r["idx"], E, None)
    s = O.balance_stats(r["scores"], "softmax", r["lse"], d["counts_pre"], d["counts_kept"], T, k, E)
    assert np.allclose(s["f"], 1.0 / E, rtol=0, atol=1e-15)
    assert np.allclose(s["P"], 1.0 / E, rtol=0, atol=1e-15)
    assert abs(s["l_aux"] - 1.0) < 1e-13
    assert s["imbalance"] == 1.0 and s["utilization"] == 1.0



@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (16, 4)])
def test_sigmoid_laux_is_one_under_uniform_routing(E, k):
    """Sigmoid router: token t's logits are a cyclic shift by t of one vector,
    T a multiple of E, so the normalised affinities s_ti / sum_e s_te average to
    1/E for every expert and the picks are uniform: P_i = f_i = 1/E, L_aux = 1.
    (Without the normalisation, P_i would be the mean of the raw sigmoids.)"""
    v = np.linspace(2.0, -1.5, E).astype(np.float32)
    T = 2 * E
    logits = np.stack([np.roll(v, t) for t in range(T)])
    r = O.route(logits, k, "sigmoid")
    d = O.dispatch(r["idx"], E, None)
    s = O.balance_stats(r["scores"], "sigmoid", r["lse"], d["counts_pre"], d["counts_kept"], T, k, E)
    assert np.allclose(s["f"], 1.0 / E, rtol=0, atol=1e-15)
    assert np.allclose(s["P"], 1.0 / E, rtol=0, atol=1e-15)
    assert abs(s["l_aux"] - 1.0) < 1e-13


def test_sigmoid_prob_mean_hand_case():
    """Two tokens, two experts, top-1, sigmoid router.
    token 0: logits (0, ln 3) -> s = (1/2, 3/4), normalised (2/5, 3/5), picks expert 1;
    token 1: logits (-ln 3, ln 3) -> s = (1/4, 3/4), normalised (1/4, 3/4), picks expert 1.
    P = ((2/5 + 1/4)/2, (3/5 + 3/4)/2) = (0.325, 0.675); f = (0, 1);
    L_aux = 2 (0 * 0.325 + 1 * 0.675) = 1.35."""
    l3 = math.log(3.0)
    logits = np.array([[0.0, l3], [-l3, l3]], np.float32)
    r = O.route(logits, 1, "sigmoid")
    assert list(r["idx"][:, 0]) == [1, 1]
    d = O.dispatch(r["idx"], 2, None)
    s = O.balance_stats(r["scores"], "sigmoid", r["lse"], d["counts_pre"], d["counts_kept"], 2, 1, 2)
    assert np.allclose(s["P"], [0.325, 0.675], rtol=0, atol=1e-7)
    assert np.array_equal(s["f"], [0.0, 1.0])
    assert s["l_aux"] == pytest.approx(1.35, abs=1e-7)
    # z-loss is the same logsumexp statistic for both routers:
    # lse(0, ln 3) = ln 4, lse(-ln 3, ln 3) = ln(10/3)
    assert s["z_loss"] == pytest.approx((math.log(4.0) ** 2 + math.log(10 / 3) ** 2) / 2, abs=1e-6)

def test_laux_all_mass_on_one_expert_is_E():
    E, T = 8, 32
    logits = np.zeros((T, E), np.float32)
    logits[:, 3] = 100.0
    r = O.route(logits, 1, "softmax")
    d = O.dispatch(r["idx"], E, None)
    s = O.balance_stats(r["scores"], "softmax", r["lse"], d["counts_pre"], d["counts_kept"], T, 1, E)
    assert abs(s["l_aux"] - E) < 1e-10
    assert s["imbalance"] == math.inf and s["utilization"] == 1.0 / E


@pytest.mark.parametrize("E", [4, 8, 256])
def test_zloss_closed_forms(E):
    T = 16
    z0 = np.zeros((T, E), np.float32)
    lse = O.logsumexp(z0)
    assert np.allclose(lse, math.log(E), rtol=0, atol=1e-14)
    r = O.route(z0, 1, "softmax")
    d = O.dispatch(r["idx"], E, None)
    s = O.balance_stats(r["scores"], "softmax", r["lse"], d["counts_pre"], d["counts_kept"], T, 1, E)
    assert abs(s["z_loss"] - math.log(E) ** 2) < 1e-12
    # a shift by c moves every logsumexp by c
    rng = np.random.default_rng(E)
    l = rng.normal(size=(T, E)).astype(np.float32)
    c = np.float32(2.5)
    assert np.allclose(O.logsumexp(l + c), O.logsumexp(l) + 2.5, rtol=0, atol=1e-6)
    # hand case: log(e^0 + e^{ln 3}) = log 4
    assert abs(O.logsumexp(np.array([[0.0, math.log(3.0)]]))[0] - math.log(4.0)) < 1e-7
    # torch's logsumexp on the same float32 logits
    assert np.allclose(O.logsumexp(l), torch.logsumexp(torch.from_numpy(l).double(), -1).numpy(),
                       rtol=1e-14, atol=0)


def test_monitoring_definitions():
    # imbalance = max/min counts, utilisation = nonzero experts / E, drop rate = dropped / total
    idx = np.array([[0], [0], [0], [0], [1], [1], [2], [2]], np.int32)
    d = O.dispatch(idx, 4, 3)
    s = O.balance_stats(np.full((8, 4), 0.25), "softmax", np.zeros(8), d["counts_pre"],
                        d["counts_kept"], 8, 1, 4)
    assert s["imbalance"] == math.inf          # expert 3 gets nothing
    assert s["utilization"] == 0.75
    assert s["dropped"] == 1 and s["kept"] == 7 and s["drop_rate"] == 1 / 8
    assert np.allclose(s["f"].sum(), 1.0)       # picks before capacity


# ---------------------------------------------------------------- dispatch
def _queue_simulation(idx, E, cap):
    """The definition as a literal per-expert queue: first choices in token order,
    then second choices, ...; an assignment joins its expert's queue if there is room."""
    T, k = idx.shape
    queues = [[] for _ in range(E)]
    for j in range(k):
        for t in range(T):
            e = int(idx[t, j])
            if cap is None or len(queues[e]) < cap:
                queues[e].append((t, j))
    assign_row = -np.ones((T, k), np.int64)
    row_token, offsets = [], [0]
    for e in range(E):
        for (t, j) in queues[e]:
            assign_row[t, j] = len(row_token)
            row_token.append(t)
        offsets.append(len(row_token))
    return assign_row, np.array(row_token, np.int64), np.array(offsets, np.int64)


@pytest.mark.parametrize("seed,T,E,k,cap", [(0, 37, 4, 2, 5), (1, 50, 8, 1, 4), (2, 64, 5, 3, 30),
                                            (3, 40, 6, 2, None), (4, 33, 3, 3, 1), (5, 1, 4, 2, 1)])
def test_dispatch_matches_queue_simulation(seed, T, E, k, cap):
    rng = np.random.default_rng(seed)
    # skewed picks so the capacity binds; distinct experts per token
    logits = (rng.normal(size=(T, E)) + np.linspace(2, -2, E)).astype(np.float32)
    idx = O.top_k(logits, k)
    d = O.dispatch(idx, E, cap)
    ar, rt, off = _queue_simulation(idx, E, cap)
    assert np.array_equal(d["assign_row"], ar)
    assert np.array_equal(d["row_token"], rt)
    assert np.array_equal(d["expert_offsets"], off)
    # invariants
    A = T * k
    assert d["counts_pre"].sum() == A
    assert d["counts_kept"].sum() + d["dropped"] == A
    want_kept = d["counts_pre"] if cap is None else np.minimum(d["counts_pre"], cap)
    assert np.array_equal(d["counts_kept"], want_kept)
    assert np.all(np.diff(d["expert_offsets"]) >= 0)
    kept = d["assign_row"] >= 0
    assert np.array_equal(np.sort(d["assign_row"][kept]), np.arange(d["expert_offsets"][-1]))
    for t, j in zip(*np.nonzero(kept)):
        r = d["assign_row"][t, j]
        assert d["row_token"][r] == t and d["row_slot"][r] == j


# ---------------------------------------------------------------- layer output
def _torch_ffn(x, w1, b1, w2, b2, act, w3=None):
    h = Fn.linear(x, w1, b1)
    if act == "gelu":
        h = Fn.gelu(h)            # exact erf form
    elif act == "relu":
        h = Fn.relu(h)
    else:
        h = Fn.silu(h) * Fn.linear(x, w3)
    return Fn.linear(h, w2, b2)


def _params(rng, E, d, F, act, bias=True, gate_bias=True, std=0.3):
    P = dict(w_gate=rng.normal(scale=std, size=(E, d)),
             b_gate=rng.normal(scale=std, size=E) if gate_bias else None,
             w1=rng.normal(scale=std, size=(E, F, d)), w2=rng.normal(scale=std, size=(E, d, F)),
             b1=rng.normal(scale=std, size=(E, F)) if bias else None,
             b2=rng.normal(scale=std, size=(E, d)) if bias else None,
             w3=rng.normal(scale=std, size=(E, F, d)) if act == "swiglu" else None)
    return P


class _W:
    def __init__(self, E, k, act="gelu", score_fn="softmax", drop=False, cf=1.0, mc=0, shared=0):
        self.num_experts, self.top_k, self.activation, self.score_fn = E, k, act, score_fn
        self.drop_tokens, self.capacity_factor, self.min_capacity = drop, cf, mc
        self.num_shared_experts = shared


def _t(a):
    return None if a is None else torch.from_numpy(np.asarray(a, np.float64))


def _torch_routing(x, P, k):
    logits = Fn.linear(_t(x), _t(P["w_gate"]), _t(P["b_gate"]))
    p = torch.softmax(logits, -1)
    g, i = torch.topk(p, k, -1)
    return p, g / g.sum(-1, keepdim=True), i


@pytest.mark.parametrize("act", ["gelu", "relu", "swiglu"])
def test_three_page_formulations_agree_with_oracle(act):
    rng = np.random.default_rng(7)
    T, d, F, E, k = 12, 6, 10, 5, 2
    x = rng.normal(size=(T, d))
    P = _params(rng, E, d, F, act, bias=act != "swiglu")
    out = O.forward(x, P, _W(E, k, act))
    _, g, i = _torch_routing(x, P, k)
    assert np.array_equal(out["idx"], i.numpy())
    def pick(name, e):
        return None if P[name] is None else _t(P[name][e])

    ffn = [lambda z, e=e: _torch_ffn(z, pick("w1", e), pick("b1", e), pick("w2", e), pick("b2", e),
                                     act, pick("w3", e))
           for e in range(E)]
    X = _t(x)
    # (1) masked loop over choice slot and expert
    y1 = torch.zeros(T, d, dtype=torch.float64)
    for j in range(k):
        for e in range(E):
            m = i[:, j] == e
            if m.any():
                y1[m] += g[m, j:j + 1] * ffn[e](X[m])
    # (2) per-token loop
    y2 = torch.zeros(T, d, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            y2[t] += g[t, j] * ffn[int(i[t, j])](X[t:t + 1])[0]
    # (3) every expert on every token, then gather the chosen ones
    allout = torch.stack([ffn[e](X) for e in range(E)], dim=1)          # [T, E, d]
    y3 = (allout[torch.arange(T)[:, None], i] * g[..., None]).sum(1)
    for yy in (y1, y2, y3):
        assert np.allclose(out["y"], yy.numpy(), rtol=1e-6, atol=1e-7)  # float32 router logits


def test_single_expert_is_dense_ffn():
    rng = np.random.default_rng(8)
    T, d, F = 9, 7, 11
    x = rng.normal(size=(T, d))
    P = _params(rng, 1, d, F, "gelu", std=0.8)
    out = O.forward(x, P, _W(1, 1, "gelu"))
    ref = _torch_ffn(_t(x), _t(P["w1"][0]), _t(P["b1"][0]), _t(P["w2"][0]), _t(P["b2"][0]), "gelu")
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(out["gates"] == 1.0)


def test_k_equals_E_is_soft_mixture():
    # with every expert selected the renormalised gates are the full softmax:
    # y = sum_i p_i E_i(x), the adaptive-mixtures combination (Moe survey, 1991 paper summary)
    rng = np.random.default_rng(9)
    T, d, F, E = 10, 5, 8, 4
    x = rng.normal(size=(T, d))
    P = _params(rng, E, d, F, "relu")
    out = O.forward(x, P, _W(E, E, "relu"))
    p = torch.softmax(Fn.linear(_t(x), _t(P["w_gate"]), _t(P["b_gate"])), -1)
    ref = sum(p[:, e:e + 1] * _torch_ffn(_t(x), _t(P["w1"][e]), _t(P["b1"][e]), _t(P["w2"][e]),
                                         _t(P["b2"][e]), "relu") for e in range(E))
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-6, atol=1e-7)  # float32 router logits


def test_capacity_drops_remove_exactly_the_overflow_terms():
    rng = np.random.default_rng(10)
    T, d, F, E, k = 40, 6, 8, 4, 2
    x = rng.normal(size=(T, d))
    P = _params(rng, E, d, F, "gelu")
    P["b_gate"] = np.array([3.0, 1.0, 0.0, -1.0])        # skew so expert 0 overflows
    w = _W(E, k, "gelu", drop=True, cf=1.0, mc=4)
    out = O.forward(x, P, w)
    cap = O.capacity(T, E, k, 1.0, 4, True)
    assert cap == 20 and out["dropped"] > 0
    ar, _, _ = _queue_simulation(out["idx"], E, cap)
    _, g, i = _torch_routing(x, P, k)
    ref = torch.zeros(T, d, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            if ar[t, j] >= 0:
                e = int(i[t, j])
                ref[t] += g[t, j] * _torch_ffn(_t(x[t:t + 1]), _t(P["w1"][e]), _t(P["b1"][e]),
                                               _t(P["w2"][e]), _t(P["b2"][e]), "gelu")[0]
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-6, atol=1e-7)  # float32 router logits
    # fully dropped tokens produce zeros
    full = np.all(out["assign_row"] < 0, axis=1)
    assert np.all(out["y"][full] == 0.0)


def test_shared_expert_adds_with_gate_one():
    rng = np.random.default_rng(11)
    T, d, F, E, k = 8, 4, 6, 6, 2
    x = rng.normal(size=(T, d))
    P = _params(rng, E, d, F, "swiglu", bias=False, gate_bias=False)
    S = _params(rng, 1, d, F, "swiglu", bias=False, gate_bias=False)
    P.update(ws1=S["w1"], ws2=S["w2"], ws3=S["w3"], bs1=None, bs2=None)
    P["e_bias"] = rng.uniform(-0.1, 0.1, size=E)
    w = _W(E, k, "swiglu", score_fn="sigmoid", shared=1)
    out = O.forward(x, P, w)
    no_shared = O.forward(x, P, _W(E, k, "swiglu", score_fn="sigmoid"))
    ref_s = _torch_ffn(_t(x), _t(S["w1"][0]), None, _t(S["w2"][0]), None, "swiglu", _t(S["w3"][0]))
    assert np.allclose(out["y"] - no_shared["y"], ref_s.numpy(), rtol=1e-10, atol=1e-12)
