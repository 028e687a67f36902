"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it stage by stage with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_38_amd import api as A
from sparse_mixture_experts_38_amd.workloads import make_inputs

# Output tolerance: max|y - r| / max|r| over the whole output.
TOL = {"f32": 1e-4, "bf16": 2e-2}
# Selection keys closer than this are near ties (both orders are correct).
TIE_MARGIN = 1e-6


class ExpertView:
    """Per-expert float64 view of a stacked [E, ...] tensor (any dtype, any device)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return self.t[e].detach().to("cpu", torch.float64).numpy()

    def __len__(self):
        return self.t.shape[0]

    @property
    def shape(self):
        return tuple(self.t.shape)


def np64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def oracle_params(inp):
    P = {}
    for n in ("w_gate", "b_gate", "e_bias"):
        P[n] = np64(inp.get(n))
    for n in ("w1", "w3", "b1", "w2", "b2", "ws1", "ws3", "bs1", "ws2", "bs2"):
        P[n] = None if inp.get(n) is None else ExpertView(inp[n])
    return P


def to_gpu(inp):
    return {k: (None if v is None else v.cuda()) for k, v in inp.items()}


def gpu_forward(w, g, cfg=None):
    """Run moe_forward on GPU inputs g; returns host copies of every output."""
    cfg = cfg or A.make_config(w)
    R = A.alloc_routing(cfg)
    stats = A.alloc_stats()
    ws = A.alloc_workspace(cfg)
    y = torch.empty(w.tokens, w.d_model, dtype=g["x"].dtype, device="cuda")
    A.forward(cfg, g["x"], A.weights_of(g), y, R, stats, ws)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in R.items() if v is not None}
    out["y"] = y.cpu()
    out["stats"] = A.read_stats(stats, w.num_experts)
    return out


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def check_route(w, x_np, P, out):
    """Logits within float32 accumulation error; top-k bit-exact on the GPU's
    logits (near ties set aside); gates and score statistics within tolerance."""
    T, E, k = w.tokens, w.num_experts, w.top_k
    ref_logits = O.router_logits(x_np, P["w_gate"], P.get("b_gate")).astype(np.float64)
    gl = out["logits"].numpy()
    scale = np.abs(ref_logits).max() + 1.0
    assert np.abs(gl - ref_logits).max() <= 2e-5 * scale, "router logits"
    r = O.route(gl, k, w.score_fn, P.get("e_bias"))
    gi = out["topk_idx"].numpy()
    bad = np.nonzero(np.any(gi != r["idx"], axis=1))[0]
    assert np.all(r["margin"][bad] < TIE_MARGIN), f"top-k differs on tokens {bad[:10]}"
    ok = np.setdiff1d(np.arange(T), bad)
    assert np.allclose(out["topk_gate"].numpy()[ok], r["gates"][ok], rtol=2e-5, atol=1e-6), "gates"
    return r, bad


def check_dispatch(w, out):
    """Counts, offsets, row maps and the drop set bit-exact given the GPU's top-k."""
    cap = O.capacity(w.tokens, w.num_experts, w.top_k, w.capacity_factor, w.min_capacity,
                     w.drop_tokens)
    d = O.dispatch(out["topk_idx"].numpy(), w.num_experts, cap)
    E, T, S = w.num_experts, w.tokens, w.num_shared_experts
    R = int(d["expert_offsets"][-1])
    off = out["expert_offsets"].numpy().astype(np.int64)
    assert np.array_equal(off[:E + 1], d["expert_offsets"]), "expert_offsets"
    if S:
        assert off[E + 1] == R + T
    assert np.array_equal(out["assign_row"].numpy(), d["assign_row"]), "assign_row"
    rt = out["row_token"].numpy()
    assert np.array_equal(rt[:R], d["row_token"]), "row_token"
    if S:
        assert np.array_equal(rt[R:R + T], np.arange(T)), "shared rows"
    st = out["stats"]
    assert np.array_equal(st["counts_pre"], d["counts_pre"])
    assert np.array_equal(st["counts_kept"], d["counts_kept"])
    assert st["kept"] == R and st["dropped"] == d["dropped"]
    assert st["capacity"] == cap
    return d


def check_layer(w, x_np, P, out, r, tol=None):
    """Layer output vs the oracle on the GPU's routing (stage isolation)."""
    ref = O.forward(x_np, P, w, logits=out["logits"].numpy(), idx=out["topk_idx"].numpy())
    err = rel_err(out["y"].float().numpy(), ref["y"])
    assert err <= (tol or TOL[w.act_dtype]), f"layer output max rel err {err}"
    st = out["stats"]
    rs = ref["stats"]
    assert np.allclose(st["prob_mean"], rs["P"], rtol=1e-4, atol=1e-7), "P_i"
    assert np.allclose(st["frac"], rs["f"], rtol=1e-6, atol=0), "f_i"
    assert abs(st["l_aux"] - rs["l_aux"]) <= 1e-4 * max(1.0, abs(rs["l_aux"])), "L_aux"
    assert abs(st["z_loss"] - rs["z_loss"]) <= 1e-4 * max(1.0, abs(rs["z_loss"])), "z-loss"
    return err


def full_check(w, seed=0):
    inp = make_inputs(w, seed=seed, device="cpu")
    g = to_gpu(inp)
    out = gpu_forward(w, g)
    x_np = np64(inp["x"])
    P = oracle_params(inp)
    r, bad = check_route(w, x_np, P, out)
    check_dispatch(w, out)
    err = check_layer(w, x_np, P, out, r)
    return out, err
