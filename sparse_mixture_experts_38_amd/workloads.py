"""Seeded synthetic inputs for the MoE-layer forward.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests. It holds only shapes, dtypes, seeds and random draws: none of
the layer's arithmetic (no capacity, routing, FFN or statistics) lives here.

Workload shapes follow the problem statements of the pages:
  * a basic layer with hidden->4*hidden GELU experts and a biased gate
    (MoE Training: Mixture of Experts, "Basic MoE Architecture");
  * DeepSpeed GPT-MoE shapes (hidden 1024, seq 2048, micro-batch 4, 8 or 128
    experts, capacity factors 1.25 train / 2.0 eval, min capacity 4)
    (MoE Training Guide, "Basic MoE Configuration" and "Core MoE Parameters");
  * Mixtral 8x7B shapes, three 4096x14336 matrices per expert and a 4096x8 gate
    (Moe(Mixtrue of Experts) survey, "How to compute training and inference
    cost" Mixtral parameter count);
  * DeepSeek-V3 fine-grained + shared experts with sigmoid scores and a
    selection bias (MoE From Scratch to DeepSeek V3, "DeepSeek Innovation" and
    "V3 key improvements").

Draw order is fixed so that every consumer sees the same values for a seed:
x, w_gate, b_gate, e_bias, then per routed expert w1, w3, b1, w2, b2, then the
shared expert's w1, w3, b1, w2, b2. Every weight is N(0, weight_std); x is
N(0, 1); b_gate is N(0, gate_bias_std); e_bias is U(-e_bias_range,
+e_bias_range). Floating tensors are drawn in float32 and then rounded
(round-to-nearest-even, torch's conversion) to the stored dtype. FFN biases,
the gate bias and the selection bias are stored in float32.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    d_model: int
    d_ff: int
    num_experts: int
    top_k: int
    score_fn: str = "softmax"          # "softmax" | "sigmoid"
    activation: str = "gelu"           # "gelu" | "relu" | "swiglu"
    has_bias: bool = True              # FFN biases b1, b2
    has_gate_bias: bool = False        # router bias b_gate
    capacity_factor: float = 1.0
    min_capacity: int = 4
    drop_tokens: bool = False
    act_dtype: str = "bf16"            # x, w1, w3, w2 and the layer output
    router_dtype: str = "f32"          # w_gate
    num_shared_experts: int = 0
    weight_std: float = 0.02
    gate_bias_std: float = 0.02
    e_bias_range: float = 0.0          # > 0 only for the sigmoid router
    description: str = ""

    def scaled(self, **changes) -> "Workload":
        """Same recipe at other sizes (for parity runs the oracle finishes quickly)."""
        name = changes.pop("name", self.name + "_scaled")
        return dataclasses.replace(self, name=name, **changes)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            "tiny_fp32", tokens=64, d_model=32, d_ff=128, num_experts=4, top_k=2,
            activation="gelu", has_bias=True, has_gate_bias=True, drop_tokens=False,
            act_dtype="f32", router_dtype="f32",
            description="T=64, d=32, 4 experts Linear(32->128)+GELU+Linear(128->32) with bias, "
                        "biased gate, softmax top-2, no capacity limit, fp32"),
        Workload(
            "deepspeed_gpt_moe", tokens=8192, d_model=1024, d_ff=4096, num_experts=8, top_k=2,
            activation="gelu", has_bias=True, has_gate_bias=False, capacity_factor=1.25,
            min_capacity=4, drop_tokens=True, act_dtype="bf16", router_dtype="f32",
            description="T=8192 (4 x 2048), d=1024, 8 experts 1024->4096 GELU ->1024, top-2 "
                        "softmax, capacity factor 1.25, min capacity 4, dropping on; bf16 "
                        "activations and experts, fp32 router"),
        Workload(
            "many_expert_train", tokens=8192, d_model=1024, d_ff=4096, num_experts=128, top_k=1,
            activation="gelu", has_bias=True, has_gate_bias=True, gate_bias_std=2.0,
            capacity_factor=1.25, min_capacity=4, drop_tokens=True, act_dtype="bf16",
            router_dtype="bf16",
            description="T=8192, d=1024, 128 experts 1024->4096 GELU ->1024, top-1 softmax, "
                        "per-expert N(0,2) logit offsets, capacity factor 1.25, min 4"),
        Workload(
            "many_expert_eval", tokens=8192, d_model=1024, d_ff=4096, num_experts=128, top_k=1,
            activation="gelu", has_bias=True, has_gate_bias=True, gate_bias_std=2.0,
            capacity_factor=2.0, min_capacity=4, drop_tokens=True, act_dtype="bf16",
            router_dtype="bf16",
            description="as many_expert_train with capacity factor 2.0"),
        Workload(
            "mixtral_8x7b", tokens=4096, d_model=4096, d_ff=14336, num_experts=8, top_k=2,
            activation="swiglu", has_bias=False, has_gate_bias=False, drop_tokens=False,
            act_dtype="bf16", router_dtype="bf16",
            description="T=4096, d=4096, 8 SwiGLU experts (w1,w3 4096->14336, w2 14336->4096), "
                        "no bias, top-2 softmax, no dropping"),
        Workload(
            "deepseek_v3", tokens=4096, d_model=7168, d_ff=2048, num_experts=256, top_k=8,
            score_fn="sigmoid", activation="swiglu", has_bias=False, has_gate_bias=False,
            drop_tokens=False, act_dtype="bf16", router_dtype="bf16", num_shared_experts=1,
            e_bias_range=0.1,
            description="T=4096, d=7168, 256 routed SwiGLU experts 7168->2048->7168 + 1 shared, "
                        "sigmoid scores + U(-0.1,0.1) selection bias, top-8"),
    ]
}

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def _normal(shape, std, gen, device, dtype):
    t = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """Draw every input of the layer for workload ``w`` (see module docstring)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    act = _DTYPES[w.act_dtype]
    T, d, F, E, S = w.tokens, w.d_model, w.d_ff, w.num_experts, w.num_shared_experts
    swiglu = w.activation == "swiglu"
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _normal((T, d), 1.0, gen, device, act)
    out["w_gate"] = _normal((E, d), w.weight_std, gen, device, _DTYPES[w.router_dtype])
    out["b_gate"] = (_normal((E,), w.gate_bias_std, gen, device, torch.float32)
                     if w.has_gate_bias else None)
    if w.e_bias_range > 0.0:
        u = torch.rand(E, generator=gen, device=device, dtype=torch.float32)
        out["e_bias"] = (u * 2.0 - 1.0) * w.e_bias_range
    else:
        out["e_bias"] = None

    def experts(n):
        w1 = torch.empty(n, F, d, device=device, dtype=act)
        w3 = torch.empty(n, F, d, device=device, dtype=act) if swiglu else None
        w2 = torch.empty(n, d, F, device=device, dtype=act)
        b1 = torch.empty(n, F, device=device, dtype=torch.float32) if w.has_bias else None
        b2 = torch.empty(n, d, device=device, dtype=torch.float32) if w.has_bias else None
        for e in range(n):
            w1[e] = _normal((F, d), w.weight_std, gen, device, act)
            if swiglu:
                w3[e] = _normal((F, d), w.weight_std, gen, device, act)
            if w.has_bias:
                b1[e] = _normal((F,), w.weight_std, gen, device, torch.float32)
            w2[e] = _normal((d, F), w.weight_std, gen, device, act)
            if w.has_bias:
                b2[e] = _normal((d,), w.weight_std, gen, device, torch.float32)
        return w1, w3, b1, w2, b2

    out["w1"], out["w3"], out["b1"], out["w2"], out["b2"] = experts(E)
    if S:
        (out["ws1"], out["ws3"], out["bs1"], out["ws2"], out["bs2"]) = experts(S)
    else:
        out["ws1"] = out["ws3"] = out["bs1"] = out["ws2"] = out["bs2"] = None
    return out


def make_x(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """Only x, drawn exactly as make_inputs draws it (it is the first draw)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return _normal((w.tokens, w.d_model), 1.0, gen, device, _DTYPES[w.act_dtype])
