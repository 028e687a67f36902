"""GPU parity of the training forward and the backward pass (through the C ABI)
against the CPU oracle.

Stage isolation: the oracle runs on the GPU's routing (logits and top-k choice),
so near ties cannot make the two sides differ in a discrete decision; the
routing itself is checked bit-exact by the forward parity tests. Every
gradient is compared over the whole tensor with the max-norm relative error
max|g - r| / max|r| against the bar of the layer's type: bf16 (the operands of
the expert GEMMs are bf16, as in the forward) or float32.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_38_amd import api as A
from sparse_mixture_experts_38_amd.workloads import WORKLOADS, make_inputs

from parity_util import TOL, check_dispatch, np64, oracle_params, rel_err, to_gpu

pytestmark = pytest.mark.gpu

W = WORKLOADS
AUX, ZC = 0.01, 0.001

CASES = {
    # DeepSpeed GPT-MoE recipe (GELU, biases, softmax top-2, capacity 1.25), ragged T
    "gpt_moe_small": W["deepspeed_gpt_moe"].scaled(tokens=1000, d_model=256, d_ff=512),
    # tight capacity so assignments are dropped
    "gpt_moe_drops": W["deepspeed_gpt_moe"].scaled(tokens=777, d_model=256, d_ff=512,
                                                   capacity_factor=0.9),
    # ReLU experts, gate bias, bf16 router weights
    "relu_bf16": W["deepspeed_gpt_moe"].scaled(tokens=333, d_model=256, d_ff=256, activation="relu",
                                               has_gate_bias=True, router_dtype="bf16"),
    # sigmoid router with selection bias, top-8 of 256, shared expert (GELU experts)
    "deepseek_small_gelu": W["deepseek_v3"].scaled(tokens=300, d_model=512, d_ff=256,
                                                   activation="gelu"),
    # 128 experts, top-1, heavy imbalance: many empty and near-empty groups
    "many_expert": W["many_expert_train"].scaled(tokens=1536, d_model=256, d_ff=256),
    # Mixtral recipe: SwiGLU experts, no biases, no capacity limit
    "mixtral_small": W["mixtral_8x7b"].scaled(tokens=700, d_model=512, d_ff=768),
    # DeepSeek-V3 recipe with its SwiGLU experts: sigmoid + selection bias, top-8 of 256, shared
    "deepseek_small": W["deepseek_v3"].scaled(tokens=300, d_model=512, d_ff=256),
    # d_model 2048: the dX GEMM takes the 256 x 256 tiles for full 256-row blocks
    "long_k": W["deepspeed_gpt_moe"].scaled(tokens=600, d_model=2048, d_ff=512, num_experts=4,
                                            drop_tokens=False),
    # the float32 layer as given (T = 64, d = 32, GELU experts with biases, gate bias)
    "tiny_fp32": W["tiny_fp32"],
    # float32 with capacity drops and ReLU
    "fp32_relu_drops": W["tiny_fp32"].scaled(tokens=97, d_model=40, d_ff=72, num_experts=5,
                                             activation="relu", drop_tokens=True,
                                             capacity_factor=0.8, min_capacity=2),
    # float32 DeepSeek-V3 recipe: sigmoid + selection bias, SwiGLU, shared expert
    "fp32_deepseek": W["deepseek_v3"].scaled(tokens=130, d_model=48, d_ff=64, num_experts=16,
                                             top_k=4, act_dtype="f32", router_dtype="f32"),
}


def gpu_train_step(w, g, dy, cfg=None, aux=AUX, zc=ZC):
    cfg = cfg or A.make_config(w)
    R = A.alloc_routing(cfg)
    stats = A.alloc_stats()
    ws = A.alloc_workspace(cfg)
    saved = A.alloc_saved(cfg)
    y = torch.empty(w.tokens, w.d_model, dtype=g["x"].dtype, device="cuda")
    A.forward_train(cfg, g["x"], A.weights_of(g), y, R, stats, saved, ws)
    grads = A.alloc_grads(cfg)
    bws = A.alloc_backward_workspace(cfg)
    A.backward(cfg, g["x"], A.weights_of(g), R, stats, saved, dy, aux, zc, grads, bws)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in R.items() if v is not None}
    out["y"] = y.cpu()
    out["stats"] = A.read_stats(stats, w.num_experts)
    out["z"] = saved["z"].cpu()
    out["y_perm"] = saved["y_perm"].cpu()
    out["grads"] = {k: (None if v is None else v.cpu()) for k, v in grads.items()}
    return out


def make_dy(w, seed, device="cpu"):
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + seed)
    dt = torch.bfloat16 if w.act_dtype == "bf16" else torch.float32
    return torch.randn(w.tokens, w.d_model, generator=gen, device=device).to(dt)


def check_backward(w, inp, dy, out):
    x_np = np64(inp["x"])
    P = oracle_params(inp)
    logits = out["logits"].numpy().astype(np.float64)
    fwd = O.forward(x_np, P, w, logits=out["logits"].numpy(), idx=out["topk_idx"].numpy())
    check_dispatch(w, out)
    tol = TOL[w.act_dtype]
    errs = {}
    # training forward: output, saved pre-activation and expert outputs
    errs["y"] = rel_err(out["y"].float().numpy(), fwd["y"])
    g = O.backward(x_np, P, w, np64(dy), AUX, ZC, fwd=fwd, logits=logits)
    R = int(fwd["expert_offsets"][-1])
    zs = out["z"].float().numpy()
    if w.activation == "swiglu":
        errs["z"] = rel_err(zs[0, :R], g["z"][:R])
        errs["u"] = rel_err(zs[1, :R], g["u"][:R])
    else:
        errs["z"] = rel_err(zs[:R], g["z"][:R])
    errs["y_perm"] = rel_err(out["y_perm"].float().numpy()[:R], fwd["Y"][:R])
    G = out["grads"]
    pairs = [("dx", "dx"), ("dw_gate", "dw_gate"), ("dw1", "dw1"), ("dw2", "dw2")]
    if w.has_bias:
        pairs += [("db1", "db1"), ("db2", "db2")]
    if w.has_gate_bias:
        pairs += [("db_gate", "db_gate")]
    if w.num_shared_experts:
        pairs += [("dws1", "dws1"), ("dws2", "dws2")]
        if w.has_bias:
            pairs += [("dbs1", "dbs1"), ("dbs2", "dbs2")]
    if w.activation == "swiglu":
        pairs += [("dw3", "dw3")] + ([("dws3", "dws3")] if w.num_shared_experts else [])
    for gk, ok in pairs:
        ref = g[ok]
        got = G[gk].float().numpy()
        assert got.shape == ref.shape, gk
        errs[gk] = rel_err(got, ref)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"max rel err above {tol}: {bad} (all: {errs})"
    return errs


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(name):
    w = CASES[name]
    print(f"[case] backward {name} T={w.tokens} d={w.d_model} F={w.d_ff} E={w.num_experts} "
          f"k={w.top_k} {w.activation} {w.score_fn}", flush=True)
    inp = make_inputs(w, seed=0, device="cpu")
    dy = make_dy(w, 0)
    out = gpu_train_step(w, to_gpu(inp), dy.cuda())
    errs = check_backward(w, inp, dy, out)
    print("  errs", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    if name == "gpt_moe_drops":
        assert out["stats"]["dropped"] > 0


def test_training_forward_matches_inference_forward():
    """moe_forward_train gives the routing of moe_forward bit for bit and the same
    output up to the bf16 rounding of the saved pre-activation."""
    w = CASES["gpt_moe_small"]
    print("[case] forward_train vs forward", flush=True)
    inp = make_inputs(w, seed=3, device="cuda")
    cfg = A.make_config(w)
    R1, R2 = A.alloc_routing(cfg), A.alloc_routing(cfg)
    s1, s2 = A.alloc_stats(), A.alloc_stats()
    ws = A.alloc_workspace(cfg)
    y1 = torch.empty(w.tokens, w.d_model, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    A.forward(cfg, inp["x"], A.weights_of(inp), y1, R1, s1, ws)
    A.forward_train(cfg, inp["x"], A.weights_of(inp), y2, R2, s2, A.alloc_saved(cfg), ws)
    torch.cuda.synchronize()
    for k in ("logits", "topk_idx", "topk_gate", "expert_offsets", "assign_row"):
        assert torch.equal(R1[k], R2[k]), k
    assert torch.equal(s1, s2)
    assert rel_err(y2.float().cpu().numpy(), y1.float().cpu().numpy()) <= 1e-2


@pytest.mark.parametrize("name", ["gpt_moe_drops", "deepseek_small"])
def test_backward_is_deterministic(name):
    """Bitwise equal gradients from two runs: the tiled kernels with capacity drops,
    and the DeepSeek-V3 recipe (K-major weight streaming for dH and dX, the router
    terms on MFMA, weight-gradient tiles of empty groups)."""
    w = CASES[name]
    print(f"[case] backward determinism {name}", flush=True)
    inp = to_gpu(make_inputs(w, seed=1, device="cpu"))
    dy = make_dy(w, 1).cuda()
    a = gpu_train_step(w, inp, dy)["grads"]
    b = gpu_train_step(w, inp, dy)["grads"]
    for k, v in a.items():
        if v is not None:
            assert torch.equal(v, b[k]), k


def test_backward_loss_coefficients_enter_linearly():
    """The gradient is linear in (dy, aux_coef, z_coef): with dy = 0 only the
    router receives a gradient, and doubling both coefficients doubles dw_gate
    and leaves the expert weights' gradients at zero."""
    w = CASES["relu_bf16"]
    print("[case] backward with dy = 0", flush=True)
    inp = to_gpu(make_inputs(w, seed=2, device="cpu"))
    dy = torch.zeros(w.tokens, w.d_model, dtype=torch.bfloat16, device="cuda")
    o1 = gpu_train_step(w, inp, dy, aux=0.01, zc=0.001)["grads"]
    o2 = gpu_train_step(w, inp, dy, aux=0.02, zc=0.002)["grads"]
    for k in ("dw1", "dw2", "db1", "db2"):
        assert float(o1[k].abs().max()) == 0.0, k
    assert float(o1["dw_gate"].abs().max()) > 0
    np.testing.assert_allclose(o2["dw_gate"].numpy(), 2 * o1["dw_gate"].numpy(), rtol=1e-5,
                               atol=1e-7 * float(o1["dw_gate"].abs().max()))


def test_backward_edge_cases():
    """One token; k = E; a single expert; every token routed to one expert (the
    other groups are empty and padded to 128 zero columns)."""
    base = W["deepspeed_gpt_moe"].scaled(d_model=256, d_ff=256)
    cases = {
        "one_token": base.scaled(tokens=1),
        "k_equals_E": base.scaled(tokens=200, num_experts=4, top_k=4, drop_tokens=False),
        "single_expert": base.scaled(tokens=150, num_experts=1, top_k=1, drop_tokens=False),
    }
    for name, w in cases.items():
        print(f"[case] backward edge {name}", flush=True)
        inp = make_inputs(w, seed=4, device="cpu")
        dy = make_dy(w, 4)
        out = gpu_train_step(w, to_gpu(inp), dy.cuda())
        check_backward(w, inp, dy, out)
    # all tokens to expert 0: a large gate bias on expert 0
    w = base.scaled(tokens=300, num_experts=8, top_k=1, has_gate_bias=True, drop_tokens=False)
    print("[case] backward edge all_to_one", flush=True)
    inp = make_inputs(w, seed=5, device="cpu")
    inp["b_gate"] = torch.zeros(8)
    inp["b_gate"][0] = 50.0
    dy = make_dy(w, 5)
    out = gpu_train_step(w, to_gpu(inp), dy.cuda())
    assert int(out["stats"]["counts_kept"][0]) == 300
    check_backward(w, inp, dy, out)


def test_backward_router_mfma_edge_cases():
    """The router terms of the backward on MFMA (bf16 router, E a multiple of
    128: dlogits as two bf16 planes, the router weight gradient over token
    slices, x's router term as a GEMM) at the token counts where the slices
    degenerate: one token, fewer tokens than one 128-row slice, and a count that
    is not a multiple of the slice size; DeepSeek-V3 recipe (sigmoid, top-8 of
    256, SwiGLU, shared expert) and a softmax router with 128 experts."""
    ds = W["deepseek_v3"].scaled(d_model=256, d_ff=256)
    cases = {
        "ds_one_token": ds.scaled(tokens=1),
        "ds_100_tokens": ds.scaled(tokens=100),
        "ds_517_tokens": ds.scaled(tokens=517),
        "softmax_128_experts": W["deepspeed_gpt_moe"].scaled(
            tokens=300, d_model=256, d_ff=256, num_experts=128, top_k=2, router_dtype="bf16",
            drop_tokens=False),
    }
    for name, w in cases.items():
        print(f"[case] backward router-mfma edge {name}", flush=True)
        inp = make_inputs(w, seed=6, device="cpu")
        dy = make_dy(w, 6)
        out = gpu_train_step(w, to_gpu(inp), dy.cuda())
        check_backward(w, inp, dy, out)


def test_backward_stream_and_tiled_groups():
    """dH and dX with one group above the streaming kernel's 1536-row limit (tiled
    kernels) and one below it (weight-streaming kernel with K-major weights) in the
    same launches: Mixtral recipe (SwiGLU, K = 2F for dX over [W1; W3]), 2 experts,
    top-1, a gate bias that sends most tokens to expert 0."""
    w = W["mixtral_8x7b"].scaled(tokens=2000, d_model=256, d_ff=512, num_experts=2, top_k=1,
                                 has_gate_bias=True)
    print("[case] backward streamed + tiled groups", flush=True)
    inp = make_inputs(w, seed=7, device="cpu")
    inp["b_gate"] = torch.tensor([0.5, 0.0])
    dy = make_dy(w, 7)
    out = gpu_train_step(w, to_gpu(inp), dy.cuda())
    kept = [int(v) for v in out["stats"]["counts_kept"][:2]]
    assert max(kept) > 1536 and min(kept) <= 1536, kept
    check_backward(w, inp, dy, out)


def test_backward_full_size_sampled():
    """DeepSpeed GPT-MoE at its full size (T = 8192, d = 1024, F = 4096, 8 experts):
    the router weight gradient in full and sampled rows of every other gradient,
    each computed by the oracle from its definition for just those entries, on
    the GPU's routing (stage isolation: logits and top-k only). The expert
    outputs Y and the pre-activations z that the reference needs are the
    oracle's own, computed from x and the weights; the GPU's saved planes are
    checked against them in full first."""
    w = W["deepspeed_gpt_moe"]
    print("[case] backward full-size deepspeed_gpt_moe", flush=True)
    inp = make_inputs(w, seed=0, device="cuda")
    dy = make_dy(w, 0, device="cuda")
    out = gpu_train_step(w, inp, dy)
    T, d, F, E, k = w.tokens, w.d_model, w.d_ff, w.num_experts, w.top_k
    x = np64(inp["x"])
    dyn = np64(dy)
    P = oracle_params(inp)
    dsp = check_dispatch(w, out)
    off = dsp["expert_offsets"]
    rt = dsp["row_token"]
    R = int(off[-1])
    # the oracle's forward on the GPU's routing: every kept row's expert output
    # Y and pre-activation z = x W1^T + b1
    Y = O.experts_forward(x, dsp, P, w.activation)
    Z = np.empty((R, F))
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            Z[lo:hi] = x[rt[lo:hi]] @ P["w1"][e].T + P["b1"][e][None, :]
    tol = TOL["bf16"]
    assert rel_err(out["z"].float().numpy()[:R], Z) <= tol, "saved z"
    assert rel_err(out["y_perm"].float().numpy()[:R], Y) <= tol, "saved y_perm"
    logits = out["logits"].numpy().astype(np.float64)
    idx = out["topk_idx"].numpy()
    # the oracle's gates on the GPU's logits and top-k
    gates = O.renormalised_gates(O.route(out["logits"].numpy(), k, w.score_fn,
                                         P.get("e_bias"))["scores"], idx)
    # combine backward on the oracle's expert outputs, then the router backward
    dYp, dgate = O.combine_backward(dyn, Y, gates, dsp["assign_row"])
    f = dsp["counts_pre"] / float(T * k)
    dlog = O.router_backward(logits, idx, w.score_fn, dgate, f, AUX, ZC)
    G = out["grads"]
    assert rel_err(G["dw_gate"].numpy(), dlog.T @ x) <= tol, "dw_gate"
    # host float64 copies of the expert weights, made once
    W1s = [P["w1"][e] for e in range(E)]
    W2s = [P["w2"][e] for e in range(E)]
    rng = np.random.default_rng(0)
    # expert gradients on sampled rows / columns of two experts
    for e in (0, E - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        W1, W2 = W1s[e], W2s[e]
        Ze = Z[lo:hi]
        He = O.gelu(Ze)
        dYe = dYp[lo:hi]
        i_s = rng.choice(d, 8, replace=False)
        f_s = rng.choice(F, 8, replace=False)
        # dW2[e][i, :] = sum_r dY[r, i] h[r, :]
        assert rel_err(G["dw2"][e].numpy()[i_s], dYe[:, i_s].T @ He) <= tol, f"dw2[{e}]"
        # dZ[:, f] = (dY W2[:, f]) * gelu'(z[:, f]); dW1[e][f, :] = sum_r dZ[r, f] x[r, :]
        dZf = (dYe @ W2[:, f_s]) * O.gelu_grad(Ze[:, f_s])
        assert rel_err(G["dw1"][e].numpy()[f_s], dZf.T @ x[rt[lo:hi]]) <= tol, f"dw1[{e}]"
        assert rel_err(G["db2"][e].numpy(), dYe.sum(axis=0)) <= tol, f"db2[{e}]"
        dZ_all = (dYe @ W2) * O.gelu_grad(Ze)
        assert rel_err(G["db1"][e].numpy(), dZ_all.sum(axis=0)) <= tol, f"db1[{e}]"
    # dx on sampled tokens (including tokens that lost a choice to capacity)
    dropped_tok = np.nonzero(np.any(dsp["assign_row"] < 0, axis=1))[0]
    toks = np.unique(np.concatenate([rng.choice(T, 48, replace=False), dropped_tok[:16]]))
    dx_ref = dlog[toks] @ P["w_gate"]
    for si, t in enumerate(toks):
        for j in range(k):
            r = dsp["assign_row"][t, j]
            if r < 0:
                continue
            e = int(idx[t, j])
            dz = (dYp[r] @ W2s[e]) * O.gelu_grad(Z[r])
            dx_ref[si] += dz @ W1s[e]
    assert rel_err(G["dx"].float().numpy()[toks], dx_ref) <= tol, "dx"


def test_backward_full_size_mixtral_sampled_tokens():
    """Mixtral 8x7B at its full size (T = 4096, d = 4096, F = 14336, 8 SwiGLU
    experts, top-2, no capacity limit), trained on a dy that is zero except on
    64 sampled tokens, with aux_coef = z_coef = 0: then only those tokens' rows
    carry gradient, so every gradient tensor has an exact reference the oracle
    computes from those rows alone (x, the weights and the GPU's routing): dx in
    full (zero off the sample), dW_g, dW1, dW3 and dW2 of every expert in full,
    and the saved planes z1, u and the expert outputs on the sampled rows."""
    w = W["mixtral_8x7b"]
    print("[case] backward full-size mixtral_8x7b (sampled tokens)", flush=True)
    inp = make_inputs(w, seed=0, device="cuda")
    T, d, F, E, k = w.tokens, w.d_model, w.d_ff, w.num_experts, w.top_k
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(T, 64, replace=False))
    gen = torch.Generator(device="cpu")
    gen.manual_seed(77)
    dy = torch.zeros(T, d, dtype=torch.bfloat16)
    dy[torch.from_numpy(sample)] = torch.randn(len(sample), d, generator=gen).to(torch.bfloat16)
    out = gpu_train_step(w, inp, dy.cuda(), aux=0.0, zc=0.0)
    x = np64(inp["x"])
    dyn = np64(dy)
    P = oracle_params(inp)
    dsp = check_dispatch(w, out)
    idx = out["topk_idx"].numpy()
    logits = out["logits"].numpy()
    gates = O.renormalised_gates(O.route(logits, k, w.score_fn)["scores"], idx)
    tol = TOL["bf16"]
    zs = out["z"].float().numpy()
    yp = out["y_perm"].float().numpy()
    # per expert, its sampled rows: the oracle's forward and backward of each row
    # (weights converted to float64 once per expert)
    pairs = [(si, j) for si in range(len(sample)) for j in range(k)]
    dgate = np.zeros((len(sample), k))
    dxp = np.zeros((len(sample), d))
    rows, z1r, ur, yr, dz1r, dur, hr, dypr, toks_of, exp_of = ([] for _ in range(10))
    for e in range(E):
        sel = [(si, j) for si, j in pairs if int(idx[sample[si], j]) == e]
        if not sel:
            continue
        W1, W3, W2 = P["w1"][e], P["w3"][e], P["w2"][e]
        ts = np.array([sample[si] for si, _ in sel])
        z1 = x[ts] @ W1.T
        u = x[ts] @ W3.T
        h = O.silu(z1) * u
        y = h @ W2.T
        g = np.array([gates[sample[si], j] for si, j in sel])
        dY = g[:, None] * dyn[ts]
        dH = dY @ W2
        dz1 = dH * u * O.silu_grad(z1)
        du = dH * O.silu(z1)
        dxe = dz1 @ W1 + du @ W3
        for q, (si, j) in enumerate(sel):
            dgate[si, j] = dyn[ts[q]] @ y[q]
            dxp[si] += dxe[q]
            rows.append(int(dsp["assign_row"][sample[si], j]))
        z1r += list(z1); ur += list(u); yr += list(y); dz1r += list(dz1); dur += list(du)
        hr += list(h); dypr += list(dY); toks_of += list(ts); exp_of += [e] * len(sel)
    rows = np.array(rows)
    assert rel_err(zs[0, rows], np.array(z1r)) <= tol, "saved z1"
    assert rel_err(zs[1, rows], np.array(ur)) <= tol, "saved u"
    assert rel_err(yp[rows], np.array(yr)) <= tol, "y_perm"
    # router: the sampled tokens alone (every other token has dgate = 0 and no
    # aux or z term)
    f = dsp["counts_pre"] / float(T * k)
    dlog = O.router_backward(logits[sample].astype(np.float64), idx[sample], w.score_fn, dgate,
                             f, 0.0, 0.0)
    G = out["grads"]
    assert rel_err(G["dw_gate"].numpy(), dlog.T @ x[sample]) <= tol, "dw_gate"
    dx_ref = np.zeros((T, d))
    dx_ref[sample] = dxp + dlog @ P["w_gate"]
    assert rel_err(G["dx"].float().numpy(), dx_ref) <= tol, "dx"
    others = np.setdiff1d(np.arange(T), sample)
    assert float(G["dx"][torch.from_numpy(others)].abs().max()) == 0.0, "dx off the sample"
    exp_of = np.array(exp_of)
    toks_of = np.array(toks_of)
    for e in range(E):
        m = exp_of == e
        xs = x[toks_of[m]]
        for name, ref in (("dw1", np.array(dz1r)[m].T @ xs), ("dw3", np.array(dur)[m].T @ xs),
                          ("dw2", np.array(dypr)[m].T @ np.array(hr)[m])):
            got = G[name][e].numpy()
            if not m.any():
                assert float(np.abs(got).max()) == 0.0, f"{name}[{e}] without rows"
                continue
            assert rel_err(got, ref) <= tol, f"{name}[{e}]"
    print(f"[case] mixtral training: {len(sample)} tokens, {len(rows)} rows checked", flush=True)


def test_backward_full_size_deepseek_v3_sampled_tokens():
    """DeepSeek-V3 layer at its full size (T = 4096, d = 7168, 256 routed SwiGLU
    experts of F = 2048 plus one shared, sigmoid + selection bias, top-8), trained
    on a dy that is zero except on 32 sampled tokens, with aux_coef = z_coef = 0:
    then only those tokens' routed rows and shared rows carry gradient, and the
    oracle computes every compared entry from those rows alone (x, the weights,
    the GPU's routing): dx in full (zero off the sample), dW_g in full, the shared
    expert's dW1, dW3, dW2 in full, and the routed experts' for four experts with
    sampled rows and two without (all zero), plus the saved planes on the sampled
    rows. The gradients stay on the GPU; only the compared tensors are copied."""
    w = W["deepseek_v3"]
    print("[case] backward full-size deepseek_v3 (sampled tokens)", flush=True)
    inp = make_inputs(w, seed=0, device="cuda")
    T, d, F, E, k = w.tokens, w.d_model, w.d_ff, w.num_experts, w.top_k
    rng = np.random.default_rng(1)
    sample = np.sort(rng.choice(T, 32, replace=False))
    gen = torch.Generator(device="cpu")
    gen.manual_seed(78)
    dy = torch.zeros(T, d, dtype=torch.bfloat16)
    dy[torch.from_numpy(sample)] = torch.randn(len(sample), d, generator=gen).to(torch.bfloat16)
    cfg = A.make_config(w)
    R = A.alloc_routing(cfg)
    stats = A.alloc_stats()
    ws = A.alloc_workspace(cfg)
    saved = A.alloc_saved(cfg)
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    A.forward_train(cfg, inp["x"], A.weights_of(inp), y, R, stats, saved, ws)
    del ws
    grads = A.alloc_grads(cfg)
    bws = A.alloc_backward_workspace(cfg)
    A.backward(cfg, inp["x"], A.weights_of(inp), R, stats, saved, dy.cuda(), 0.0, 0.0, grads, bws)
    torch.cuda.synchronize()
    del bws
    out = {n: v.cpu() for n, v in R.items() if v is not None}
    out["stats"] = A.read_stats(stats, E)
    dsp = check_dispatch(w, out)
    idx = out["topk_idx"].numpy()
    logits = out["logits"].numpy()
    gates = O.renormalised_gates(O.route(logits, k, w.score_fn)["scores"], idx)
    off = out["expert_offsets"].numpy().astype(np.int64)
    x = np64(inp["x"][torch.from_numpy(sample).cuda()])   # the sampled tokens' rows
    dys = np64(dy[torch.from_numpy(sample)])
    P = oracle_params(inp)
    tol = TOL["bf16"]

    def ffn(W1, W3, W2, xs, dY):
        z1, u = xs @ W1.T, xs @ W3.T
        h = O.silu(z1) * u
        dH = dY @ W2
        dz1, du = dH * u * O.silu_grad(z1), dH * O.silu(z1)
        return z1, u, h @ W2.T, dz1 @ W1 + du @ W3, dz1.T @ xs, du.T @ xs, dY.T @ h

    dgate = np.zeros((len(sample), k))
    dxp = np.zeros((len(sample), d))
    ref_w = {}
    check_experts = []
    rows_z1, rows_ref = [], []
    zplanes = saved["z"]
    by_expert = {}
    for si in range(len(sample)):
        for j in range(k):
            by_expert.setdefault(int(idx[sample[si], j]), []).append((si, j))
    with_rows = sorted(by_expert)
    check_experts = with_rows[:: max(1, len(with_rows) // 4)][:4]
    without = [e for e in range(E) if e not in by_expert][:2]
    for e, sel in by_expert.items():
        sis = np.array([si for si, _ in sel])
        g = np.array([gates[sample[si], j] for si, j in sel])
        z1, u, ye, dxe, dw1, dw3, dw2 = ffn(P["w1"][e], P["w3"][e], P["w2"][e], x[sis],
                                            g[:, None] * dys[sis])
        for q, (si, j) in enumerate(sel):
            dgate[si, j] = dys[si] @ ye[q]
            dxp[si] += dxe[q]
        if e in check_experts:
            ref_w[e] = (dw1, dw3, dw2)
            rows = [int(dsp["assign_row"][sample[si], j]) for si, j in sel]
            rows_z1.append((rows, z1, u))
    # shared expert: every sampled token's shared row (gate 1)
    s1, s3, s2 = (np64(inp[n].reshape(inp[n].shape[-2:])) for n in ("ws1", "ws3", "ws2"))
    z1s, us, _, dxs, dws1, dws3, dws2 = ffn(s1, s3, s2, x, dys)
    dxp += dxs
    srows = off[E] + sample
    del s1, s3, s2
    for rows, z1, u in rows_z1 + [(list(srows), z1s, us)]:
        ridx = torch.tensor(rows, dtype=torch.long, device="cuda")
        assert rel_err(zplanes[0][ridx].float().cpu().numpy(), z1) <= tol, "saved z1"
        assert rel_err(zplanes[1][ridx].float().cpu().numpy(), u) <= tol, "saved u"
    f = dsp["counts_pre"] / float(T * k)
    dlog = O.router_backward(logits[sample].astype(np.float64), idx[sample], w.score_fn, dgate,
                             f, 0.0, 0.0)
    assert rel_err(grads["dw_gate"].cpu().numpy(), dlog.T @ x) <= tol, "dw_gate"
    dx = grads["dx"].float().cpu().numpy()
    assert rel_err(dx[sample], dxp + dlog @ P["w_gate"]) <= tol, "dx"
    others = np.setdiff1d(np.arange(T), sample)
    assert float(np.abs(dx[others]).max()) == 0.0, "dx off the sample"
    for name, ref in (("dws1", dws1), ("dws3", dws3), ("dws2", dws2)):
        assert rel_err(grads[name].cpu().numpy(), ref) <= tol, name
    for e in check_experts:
        for name, ref in zip(("dw1", "dw3", "dw2"), ref_w[e]):
            assert rel_err(grads[name][e].cpu().numpy(), ref) <= tol, f"{name}[{e}]"
    for e in without:
        for name in ("dw1", "dw3", "dw2"):
            assert float(grads[name][e].abs().max()) == 0.0, f"{name}[{e}] without rows"
    print(f"[case] deepseek_v3 training: {len(sample)} tokens, {len(by_expert)} routed experts, "
          f"checked {check_experts} and {without}", flush=True)
