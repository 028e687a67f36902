#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X, with the grouped expert GEMMs
measured against their roofline and the CPU oracle timed beside it.

One step = the whole forward (router + top-k, capacity dispatch, grouped GEMM 1
with the fused row gather and activation, grouped GEMM 2, weighted combine,
statistics) over one batch of synthetic tokens already resident in HBM,
through the library's forward entry point on one stream. Each step is the
event-bracketed variant moe_forward_profiled (the same kernels with the same
arguments as moe_forward, plus a HIP event at every stage boundary on the
launch stream), so the grouped GEMMs are timed exactly as they run inside the
timed forward. Input and weight sets are rotated so the 256 MB Infinity Cache
does not hold the previous step's operands.

The headline workload is the DeepSeek-V3-shaped layer (256 routed SwiGLU
experts + 1 shared, top-8 sigmoid, d 7168), the largest of the layers the
pages describe that fits one GPU. Its grouped GEMMs stream 16+ GB of expert
weights per step at about 190 FLOP per byte, below the chip's ridge point
(2.5 PFLOP/s / 8 TB/s = 312 FLOP/B), so the roofline is HBM. The roofline
bound is chosen per workload from the dominant GEMM's algorithmic FLOP per
algorithmic byte. Other workloads, one training step and expert-choice routing
are reported as extra keys. Prints one JSON line.
"""
import argparse
import ctypes
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer forward tokens/sec on 1 MI355X; grouped-GEMM % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # FLOP per byte
COPY_BYTES = 256 << 20      # each of read and write for the calibration copy
GEMM_SOURCE = os.path.join(ROOT, "sparse_mixture_experts_38_amd", "csrc", "expert_gemm.hip")
EXTRA_WORKLOADS = ("deepspeed_gpt_moe", "mixtral_8x7b")
SECONDARY = "deepspeed_gpt_moe"   # workload of the training and expert-choice figures
TRAIN_LARGE = "mixtral_8x7b"     # a second training figure at a large dense-expert layer


def kernel_source_hash():
    return hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()[:16]


def read_traffic(stage, workload):
    """HBM bytes per launch of a GEMM stage from the committed rocprofv3 counter
    summary for this workload, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"expert_gemm_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != kernel_source_hash():
        return None
    v = vals.get(f"{stage}_hbm_bytes_per_launch")
    return float(v) if v else None


def gemm_work(w, counts_kept):
    """Algorithmic FLOP and HBM bytes of the two grouped-GEMM stages.

    Rows: the kept routed rows R (+ T shared rows). FLOP: 2 rows d F per
    matrix product (GEMM 1 has two for SwiGLU). Bytes, what the stage must
    move at least: the weights (and biases) of every group that received rows,
    each read once; GEMM 1 reads x once (its row gather may revisit a token for
    each of its k choices, from cache) and writes H [rows, F]; GEMM 2 reads H
    and writes y_perm [rows, d]."""
    b = 2 if w.act_dtype == "bf16" else 4
    T, d, F, S = w.tokens, w.d_model, w.d_ff, w.num_shared_experts
    R = int(sum(counts_kept))
    used = int(sum(1 for c in counts_kept if c > 0)) + S
    rows = R + S * T
    mats_up = 2 if w.activation == "swiglu" else 1
    bias_up = F * 4 if w.has_bias else 0
    bias_dn = d * 4 if w.has_bias else 0
    up = {"flop": 2.0 * rows * d * F * mats_up,
          "bytes": used * (mats_up * F * d * b + bias_up) + T * d * b + rows * F * b}
    down = {"flop": 2.0 * rows * F * d,
            "bytes": used * (d * F * b + bias_dn) + rows * F * b + rows * d * b}
    return {"expert_up": up, "expert_down": down, "rows": rows, "groups_with_rows": used}


def roofline(w, work, stage_ms, packed=True):
    """Roofline of the longer GEMM stage: bound by its algorithmic intensity.
    The counter bytes (traffic) were taken on the packed weights; for the
    standard layout they are not known (null)."""
    dom = max(("expert_up", "expert_down"), key=lambda s: stage_ms[s])
    flop, byts, ms = work[dom]["flop"], work[dom]["bytes"], stage_ms[dom]
    intensity = flop / byts
    mfma = {"achieved": flop / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    hbm = {"achieved": byts / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    r = hbm if intensity < RIDGE else mfma
    out = {"bound": "hbm" if intensity < RIDGE else "mfma", "kernel": dom,
           "achieved": r["achieved"], "peak": r["peak"], "unit": r["unit"],
           "frac": r["achieved"] / r["peak"],
           "traffic": read_traffic(dom, w.name) if packed else None,
           "algorithmic_bytes": byts, "algorithmic_flop": flop,
           "intensity_flop_per_byte": intensity, "stage_ms": ms}
    # the other roofline of the same stage, for context
    other = mfma if r is hbm else hbm
    out["other"] = {"achieved": other["achieved"], "peak": other["peak"], "unit": other["unit"],
                    "frac": other["achieved"] / other["peak"]}
    return out


def measure_forward(A, torch, w, n_sets, steps, warmup, packed=True):
    """Times `steps` event-bracketed forward steps of workload w over rotated
    input sets; returns per-step and per-stage medians and the GEMM roofline.
    With `packed`, each set's expert weights are also given in the packed order
    of the weight-streaming GEMM (moe_pack_weights, run once per set before any
    timing: a load-time conversion of the parameters, like storing a
    checkpoint in the kernel's layout)."""
    from sparse_mixture_experts_38_amd.workloads import make_inputs
    cfg = A.make_config(w)
    sets = [make_inputs(w, seed=s, device="cuda") for s in range(n_sets)]
    if packed and w.act_dtype == "bf16":
        for st in sets:
            st.update({k: v for k, v in A.pack_weights(cfg, A.weights_of(st)).items()
                       if k in ("up_packed", "down_packed")})
        torch.cuda.synchronize()
    T, d = w.tokens, w.d_model
    act = A.TORCH_DTYPE[cfg.act_dtype]
    ws = A.alloc_workspace(cfg)
    plans = []
    for s in sets:
        R = A.alloc_routing(cfg, logits=False)
        stats = A.alloc_stats()
        y = torch.empty(T, d, dtype=act, device="cuda")
        plans.append(A.Plan(cfg, s["x"], A.weights_of(s), y, R, stats, ws))
    nev = len(A.FORWARD_EVENTS)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    for row in evs:   # create the HIP events
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(warmup):
        plans[i % len(plans)].forward_profiled(evs[0])
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        plans[i % len(plans)].forward_profiled(evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_ms = start.elapsed_time(stop) / steps
    names = A.FORWARD_EVENTS

    def med(a, b):
        ia, ib = names.index(a), names.index(b)
        return statistics.median(e[ia].elapsed_time(e[ib]) for e in evs)

    step_ms = med("start", "end")
    stage_ms = {"route": med("start", "routed"), "dispatch": med("routed", "dispatched"),
                "expert_up": med("dispatched", "up"), "expert_down": med("up", "down"),
                "combine": med("down", "end")}
    kept = [A.read_stats(p.keep[4], w.num_experts)["counts_kept"] for p in plans]
    # algorithmic work averaged over the rotated sets (their routings differ)
    works = [gemm_work(w, kc) for kc in kept]
    work = {st: {q: statistics.mean(x[st][q] for x in works) for q in ("flop", "bytes")}
            for st in ("expert_up", "expert_down")}
    work["groups_with_rows"] = statistics.mean(x["groups_with_rows"] for x in works)
    res = {"ms_per_step": step_ms, "ms_per_step_mean": mean_ms, "tokens_per_s": T / (step_ms * 1e-3),
           "weights": "packed" if "up_packed" in sets[0] else "standard",
           "stages_ms": stage_ms, "kept_rows": statistics.mean(int(sum(kc)) for kc in kept),
           "groups_with_rows": work["groups_with_rows"], "wall_s": wall,
           "roofline": roofline(w, work, stage_ms, packed="up_packed" in sets[0])}
    return res, cfg, sets, ws


def cpu_baseline(w, inp_gpu, max_seconds=30.0):
    """The oracle, as it stands, on a sample of the same workload's batch: the
    first n tokens (for a layer without a capacity limit each token's output is
    the one it has in the full batch), with n sized so one run takes about
    10-30 s on the host's cores."""
    import numpy as np
    import torch
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1

    def f64(t):
        return None if t is None else t.detach().to("cpu", torch.float64).numpy()

    class PerExpert:
        def __init__(self, t):
            self.t = t.cpu()

        def __getitem__(self, e):
            return self.t[e].to(torch.float64).numpy()

    P = {n: f64(inp_gpu[n]) for n in ("w_gate", "b_gate", "e_bias")}
    P.update({n: (None if inp_gpu[n] is None else PerExpert(inp_gpu[n]))
              for n in ("w1", "w3", "b1", "w2", "b2", "ws1", "ws3", "bs1", "ws2", "bs2")})
    x = f64(inp_gpu["x"])
    # tokens per run, from the oracle's active work: a full-batch run for the
    # small layers, a 512-token sample for the 256-expert layer
    n = w.tokens if w.tokens * w.top_k * w.d_model * w.d_ff <= 8192 * 2 * 1024 * 4096 else 512
    n = min(n, w.tokens)
    ws = w.scaled(name=w.name, tokens=n)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        O.forward(x[:n], P, ws)
        times.append(time.perf_counter() - t0)
        spent = time.perf_counter() - t_start
        if spent >= 10.0 or spent + times[-1] > max_seconds:
            break
    med = statistics.median(times)
    what = (f"full {w.name} batch ({n} tokens)" if n == w.tokens else
            f"first {n} tokens of the {w.name} batch (no capacity limit: outputs as in the full batch)"
            if not w.drop_tokens else f"first {n} tokens of the {w.name} batch")
    return {"value": n / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, numpy float64 oracle, median of {len(times)} run(s), {med:.2f} s each"}


def expert_choice_step(A, torch, w, cfg, sets, steps, warmup):
    """The same layer with expert-choice routing (moe_forward_expert_choice): every
    expert takes C tokens, so its GEMMs run on E C rows (algorithmic FLOPs
    2 x 2 E C d F)."""
    T, d, F, E = w.tokens, w.d_model, w.d_ff, w.num_experts
    act = A.TORCH_DTYPE[cfg.act_dtype]
    C = A.expert_choice_capacity(cfg)
    ws = A.alloc_ec_workspace(cfg)
    plans = [A.EcPlan(cfg, s["x"], A.weights_of(s), torch.empty(T, d, dtype=act, device="cuda"),
                      A.alloc_ec_routing(cfg, logits=False), A.alloc_stats(), ws) for s in sets]
    for i in range(warmup):
        plans[i % len(plans)].forward()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        plans[i % len(plans)].forward()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = statistics.median(e[0].elapsed_time(e[1]) for e in ev)
    st = A.read_stats(plans[0].keep[5], E)
    flop = 2 * 2.0 * E * C * d * F * (1.5 if w.activation == "swiglu" else 1.0)
    return {"workload": w.name, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "capacity": C,
            "expert_rows": E * C, "unpicked_tokens": st["dropped"],
            "gemm_tflops_over_step": flop / (ms * 1e-3) / 1e12}


def train_step(A, torch, w, cfg, sets, ws, steps, warmup, rows):
    """One training step of the layer: moe_forward_train then moe_backward (with
    L_aux and z-loss weights 0.01 and 0.001), on the same rotated input sets.
    The backward's algorithmic FLOPs are its expert GEMMs, 4 x 2 R d F (dH and
    dX, dW2 and dW1; 6 x 2 R d F for SwiGLU: dX at K = 2F and dW3), R = kept rows.
    The weights are read in their standard layout only: an optimizer step
    changes them every step, so a packed copy would have to be rebuilt each
    time (the forward figures use it as a stored layout of fixed weights)."""
    T, d, F = w.tokens, w.d_model, w.d_ff
    act = A.TORCH_DTYPE[cfg.act_dtype]
    grads = A.alloc_grads(cfg)
    bws = A.alloc_backward_workspace(cfg)
    tplans = []
    for i, s in enumerate(sets):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1000 + i)
        dy = torch.randn(T, d, generator=gen, device="cuda").to(act)
        R = A.alloc_routing(cfg)
        wstd = {k: (None if k in ("up_packed", "down_packed") else v)
                for k, v in A.weights_of(s).items()}
        tplans.append(A.TrainPlan(cfg, s["x"], wstd, torch.empty(T, d, dtype=act, device="cuda"),
                                  R, A.alloc_stats(), A.alloc_saved(cfg), ws, dy, grads, bws))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(warmup):
        p = tplans[i % len(tplans)]
        p.forward()
        p.backward()
    torch.cuda.synchronize()
    for i in range(steps):
        p = tplans[i % len(tplans)]
        ev[i][0].record()
        p.forward()
        ev[i][1].record()
        p.backward()
        ev[i][2].record()
    torch.cuda.synchronize()
    step_ms = statistics.median(e[0].elapsed_time(e[2]) for e in ev)
    fwd_ms = statistics.median(e[0].elapsed_time(e[1]) for e in ev)
    bwd_ms = statistics.median(e[1].elapsed_time(e[2]) for e in ev)
    # dH and dX (K = 2F for SwiGLU), dW2 and dW1 (+ dW3 for SwiGLU)
    bwd_flop = (6 if w.activation == "swiglu" else 4) * 2.0 * rows * d * F
    tf = bwd_flop / (bwd_ms * 1e-3) / 1e12
    return {"workload": w.name, "weights": "standard", "step_ms": step_ms, "forward_train_ms": fwd_ms,
            "backward_ms": bwd_ms, "tokens_per_s": T / (step_ms * 1e-3),
            "backward_gemm_flop": bwd_flop, "backward_tflops": tf,
            "backward_frac_of_peak": tf / PEAK_BF16_TFLOPS, "aux_coef": 0.01, "z_coef": 0.001}


def release(torch):
    """Return the device memory of the buffers the caller has dropped."""
    gc.collect()
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek_v3")
    ap.add_argument("--sets", type=int, default=2, help="rotated input/weight sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline workload's forward (no other workloads, training or expert choice)")
    ap.add_argument("--no-expert-choice", action="store_true")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-standard-layout", action="store_true",
                    help="skip the second measurement with the weights in the standard layout only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB float32 copy kernel (torch.neg) three times, "
                         "so that hardware byte counters can be scaled by a kernel of known traffic")
    ap.add_argument("--only", choices=("train", "expert_choice"),
                    help="measure only the training step or only expert-choice routing of "
                         "--workload (after a short forward measurement that sets them up) and "
                         "print that figure as a JSON line; for focused kernel traces")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer runs "
              "with all experts on one MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_mixture_experts_38_amd import api as A
    from sparse_mixture_experts_38_amd.workloads import WORKLOADS

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = COPY_BYTES // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    w = WORKLOADS[args.workload]
    if args.only:
        head, cfg, sets, ws = measure_forward(A, torch, w, args.sets, 2, 1)
        if args.only == "train":
            r = train_step(A, torch, w, cfg, sets, ws, args.steps, args.warmup, head["kept_rows"])
        else:
            r = expert_choice_step(A, torch, w, cfg, sets, args.steps, args.warmup)
        print(json.dumps({"only": args.only, **r}), flush=True)
        return
    head, cfg, sets, ws = measure_forward(A, torch, w, args.sets, args.steps, args.warmup)
    T, d, F, E, k = w.tokens, w.d_model, w.d_ff, w.num_experts, w.top_k
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.act_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "d_model": d, "d_ff": F, "num_experts": E,
                   "num_shared_experts": w.num_shared_experts, "top_k": k,
                   "activation": w.activation, "score_fn": w.score_fn,
                   "capacity_factor": w.capacity_factor if w.drop_tokens else None,
                   "min_capacity": w.min_capacity if w.drop_tokens else None,
                   "drop_tokens": w.drop_tokens, "router_dtype": w.router_dtype,
                   "parallelism": "single-gpu", "rotated_sets": args.sets},
        "roofline": head["roofline"],
        "weights": head["weights"],
        "ms_per_step_mean": head["ms_per_step_mean"],
        "stages_ms": head["stages_ms"],
        "kept_rows": head["kept_rows"],
        "groups_with_rows": head["groups_with_rows"],
        "wall_s": head["wall_s"],
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, sets[0])
    if not args.no_train and not args.no_extras and A.lib().moe_backward_workspace_size(
            ctypes.byref(cfg), ctypes.byref(ctypes.c_size_t(0))) == A.MOE_OK:
        # a training step of the headline layer itself
        result["train_" + w.name] = train_step(A, torch, w, cfg, sets, ws, max(5, args.steps // 4),
                                               2, head["kept_rows"])
    sets = ws = None
    release(torch)
    if head["weights"] == "packed" and not args.no_standard_layout:
        # the same layer with the weights in the standard [out, in] layout only
        r, _, sx, wx = measure_forward(A, torch, w, args.sets, args.steps, args.warmup, packed=False)
        result["standard_layout"] = {k2: r[k2] for k2 in ("ms_per_step", "tokens_per_s", "stages_ms",
                                                           "roofline")}
        sx = wx = None
        release(torch)
    if not args.no_extras:
        result["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            if name == w.name:
                continue
            wx = WORKLOADS[name]
            steps = max(5, args.steps)
            r, cfgx, setsx, wsx = measure_forward(A, torch, wx, args.sets, steps, args.warmup)
            result["workloads"][name] = {k2: r[k2] for k2 in ("ms_per_step", "tokens_per_s", "weights",
                                                               "stages_ms", "kept_rows", "roofline")}
            if name == SECONDARY:
                if not args.no_expert_choice and A.lib().moe_expert_choice_workspace_size(
                        ctypes.byref(cfgx), ctypes.byref(ctypes.c_size_t(0))) == A.MOE_OK:
                    result["expert_choice"] = expert_choice_step(A, torch, wx, cfgx, setsx, steps,
                                                                 args.warmup)
                if not args.no_train and A.lib().moe_backward_workspace_size(
                        ctypes.byref(cfgx), ctypes.byref(ctypes.c_size_t(0))) == A.MOE_OK:
                    result["train"] = train_step(A, torch, wx, cfgx, setsx, wsx, steps, args.warmup,
                                                 r["kept_rows"])
            if name == TRAIN_LARGE and not args.no_train:
                result["train_" + name] = train_step(A, torch, wx, cfgx, setsx, wsx, max(5, steps // 4),
                                                     2, r["kept_rows"])
            setsx = wsx = None
            release(torch)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
