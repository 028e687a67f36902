"""The allocation-free forward (moe_forward_noalloc: the library's static
per-GPU workspace) against moe_forward with a caller workspace, through the C
ABI: two calls in a row on the same GPU, the second with a smaller layer, so
the second call runs on the buffer the first one left behind."""
import ctypes

import pytest
import torch

from sparse_mixture_experts_38_amd import api as A
from sparse_mixture_experts_38_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _run(w, noalloc):
    cfg = A.make_config(w)
    inp = {k: (None if v is None else v.cuda()) for k, v in make_inputs(w, seed=3).items()}
    R = A.alloc_routing(cfg)
    stats = A.alloc_stats()
    y = torch.empty(w.tokens, w.d_model, dtype=inp["x"].dtype, device="cuda")
    if noalloc:
        A.forward_noalloc(cfg, inp["x"], A.weights_of(inp), y, R, stats)
    else:
        A.forward(cfg, inp["x"], A.weights_of(inp), y, R, stats, A.alloc_workspace(cfg))
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in R.items() if v is not None}
    out["y"] = y.cpu()
    out["stats"] = stats.cpu()
    return out


def test_forward_noalloc_matches_forward_twice():
    base = WORKLOADS["deepseek_v3"].scaled(d_model=512, d_ff=256)
    for T in (1200, 333):   # the second call is smaller and reuses the first one's buffer
        w = base.scaled(tokens=T)
        print(f"[case] noalloc T={T}", flush=True)
        assert A.workspace_size(A.make_config(w)) <= A.NOALLOC_WORKSPACE_BYTES
        ref = _run(w, noalloc=False)
        got = _run(w, noalloc=True)
        for k in ref:
            assert torch.equal(ref[k], got[k]), (T, k)   # same kernels: bitwise equal


def test_forward_noalloc_refuses_layers_over_the_limit():
    w = WORKLOADS["deepseek_v3"]    # 653 MiB of workspace
    cfg = A.make_config(w)
    assert A.workspace_size(cfg) > A.NOALLOC_WORKSPACE_BYTES
    lib = A.lib()
    assert lib.moe_forward_noalloc(ctypes.byref(cfg), None, None, None, None, None, None) == \
        A.MOE_ERR_WORKSPACE
