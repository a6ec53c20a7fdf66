"""moe_expert_ffn_noalloc (h in the library's static device scratch, for
callers that cannot allocate) against moe_expert_ffn (h in a caller
workspace), through the C ABI: two calls in a row on one GPU, the second with
a smaller input, each bit-identical to the workspace entry point on the same
inputs and, like it, within the bar of the oracle's FFN rows; shapes whose h
exceeds the scratch are rejected before any launch."""
import numpy as np
import pytest
import torch

import oracle
import mixture_experts_layer_07_amd as moe
from mixture_experts_layer_07_amd import binding
from mixture_experts_layer_07_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 3e-2}


def case(name, cid, T, act="bf16", wdt="bf16"):
    return wl.Workload(name, cid, T=T, H=384, E=24, I=256, k=4, method=wl.ROUTE_DEEPSEEKV3,
                       n_group=4, topk_group=2, scaling=2.5, bias=True, n_shared=1, act=act, wdt=wdt)


def run_pair(w, seed):
    """(noalloc fc2_out, workspace fc2_out, oracle rows) for one input."""
    inp = wl.make_inputs(w, seed)
    ids, _, _ = oracle.route(inp["logits"], w.k, w.method, w.n_group, w.topk_group, inp["bias"],
                             w.scaling, False)
    off, pp, _ = oracle.permute(ids, w.E, w.n_shared)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    off_d, pp_d = torch.from_numpy(off).to(DEV), torch.from_numpy(pp).to(DEV)
    a = moe.expert_ffn_noalloc(g["x"], off_d, pp_d, g["w13"], g["w2"], w.k, w.E, w.n_shared,
                               g["w13_scale"], g["w2_scale"])
    torch.cuda.synchronize()
    b = moe.expert_ffn(g["x"], off_d, pp_d, g["w13"], g["w2"], w.k, w.E, w.n_shared,
                       g["w13_scale"], g["w2_scale"])
    torch.cuda.synchronize()
    W = oracle.Weights(inp["w13"], inp["w2"], w.wdt, inp["w13_scale"], inp["w2_scale"])
    ref = oracle.expert_rows(W, inp["x"], w.act, w.T, w.k, w.E, w.n_shared, off, pp,
                             np.arange(w.R, dtype=np.int32))
    return a, b, ref


@pytest.mark.parametrize("act,wdt", [("bf16", "bf16"), ("bf16", "fp8"), ("f32", "f32")])
def test_noalloc_matches_workspace_entry_two_calls(act, wdt):
    big = case(f"noalloc_big_{wdt}", 97, T=300, act=act, wdt=wdt)
    small = case(f"noalloc_small_{wdt}", 98, T=37, act=act, wdt=wdt)
    for w, seed in ((big, 5), (small, 6)):   # the second call: fewer rows, other values
        print(f"noalloc case {w.name} T={w.T} act={act} wdt={wdt}", flush=True)
        a, b, ref = run_pair(w, seed)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{w.name}: differs from moe_expert_ffn"
        got = a.double().cpu().numpy()
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err < TOL[wdt], f"{w.name}: rel L2 {err} vs the oracle"


def test_noalloc_rejects_h_beyond_scratch_on_gpu():
    """h of (T*k + n_shared*T) x I values above the static scratch: MOE_ERR_UNSUPPORTED
    before any launch (the pointers are never dereferenced)."""
    L = moe.lib()
    p = torch.empty(16, dtype=torch.uint8, device=DEV)
    I, k, n_shared = 2048, 8, 1
    T = binding.NOALLOC_SCRATCH_BYTES // ((k + n_shared) * I * 2) + 1
    st = L.moe_expert_ffn_noalloc(p.data_ptr(), binding.BF16, T, 7168, I, k, 256, n_shared,
                                  p.data_ptr(), p.data_ptr(), p.data_ptr(), p.data_ptr(),
                                  binding.BF16, None, None, p.data_ptr(), None)
    assert st == 2, (st, binding.last_error())
    assert "static scratch" in binding.last_error()
