"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: routing ids, permutation, unpermute and offsets bit-exact; scales within
1e-6 relative; layer output relative L2 error within 1e-5 (fp32), 1e-2 (bf16
activations and weights), 3e-2 (fp8 weights).  Every input comes from the
seeded workload generator; every expected value from the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import mixture_experts_layer_07_amd as moe
from mixture_experts_layer_07_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {("f32", "f32"): 1e-5, ("bf16", "bf16"): 1e-2, ("bf16", "fp8"): 3e-2}


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def host(t):
    return t.detach().cpu()


def oracle_route(w, logits, bias):
    return oracle.route(logits, w.k, w.method, w.n_group, w.topk_group, bias, w.scaling,
                        bool(w.flags & wl.ROUTE_FLAG_RENORMALIZE))


def gpu_route(w, logits, bias):
    return moe.route(logits.to(DEV), w.k, w.method, w.n_group, w.topk_group,
                     None if bias is None else bias.to(DEV), w.scaling,
                     bool(w.flags & wl.ROUTE_FLAG_RENORMALIZE))


def check_route(w, logits, bias):
    ids_g, sc_g = gpu_route(w, logits, bias)
    ids_o, sc_o, hard = oracle_route(w, logits, bias)
    assert hard == 0, f"{hard} sigmoid values within rounding distance of an fp32 midpoint"
    ids_g = host(ids_g).numpy()
    assert np.array_equal(ids_g, ids_o), f"ids differ in {np.sum(np.any(ids_g != ids_o, 1))} rows"
    sc_g = host(sc_g).numpy().astype(np.float64)
    rel = np.abs(sc_g - sc_o) / np.maximum(np.abs(sc_o), 1e-300)
    assert rel.max() <= 1e-6, f"scale rel err {rel.max()}"
    return ids_o, sc_o


def check_permute(ids, E, n_shared):
    T, k = ids.shape
    off_g, pp_g, up_g = moe.permute(torch.from_numpy(ids).to(DEV), E, n_shared)
    off_o, pp_o, up_o = oracle.permute(ids, E, n_shared)
    assert np.array_equal(host(off_g).numpy(), off_o)
    assert np.array_equal(host(pp_g).numpy(), pp_o)
    assert np.array_equal(host(up_g).numpy(), up_o)
    return off_o, pp_o, up_o


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_route_parity_workloads(name):
    w = wl.WORKLOADS[name]
    x = wl.make_x(w)
    check_route(w, wl.make_logits(w, x), wl.make_bias(w))


TIE_GRID = np.array([-2, -1, 0, 1, 2], np.float32) / np.float32(4)


@pytest.mark.parametrize("E,k,method,n_group,topk_group", [
    (8, 2, 0, 1, 1), (8, 8, 0, 1, 1), (64, 6, 1, 1, 1), (65, 3, 4, 1, 1), (256, 8, 4, 1, 1),
    (128, 8, 0, 1, 1), (256, 8, 2, 8, 4), (256, 1, 2, 8, 1), (64, 8, 2, 32, 4),
    (256, 8, 2, 128, 8), (96, 5, 2, 3, 2), (12, 4, 2, 6, 3), (256, 8, 2, 16, 16),
    (256, 8, 2, 4, 2), (64, 4, 2, 2, 1), (48, 4, 2, 8, 3),
    (8, 1, 3, 1, 1), (128, 4, 3, 1, 1), (64, 8, 5, 1, 1), (256, 8, 5, 1, 1),
    (32, 4, 6, 1, 1), (256, 8, 6, 1, 1), (7, 7, 6, 1, 1),
])
@pytest.mark.parametrize("ties", [True, False])
def test_route_parity_fuzz(E, k, method, n_group, topk_group, ties):
    rng = np.random.default_rng(E * 1000 + k * 10 + method + int(ties))
    T = 333
    if ties:
        logits = rng.choice(TIE_GRID, size=(T, E)).astype(np.float32)
        bias = (rng.choice(TIE_GRID, size=E) / np.float32(2)).astype(np.float32)
    else:
        logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
        bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    w = wl.Workload("fuzz", 98, T=T, H=128, E=E, I=128, k=k, method=method,
                    flags=int(rng.integers(0, 2)), n_group=n_group, topk_group=topk_group,
                    scaling=float(rng.choice([1.0, 2.5])), bias=method in (2, 5))
    check_route(w, torch.from_numpy(logits), torch.from_numpy(bias) if w.bias else None)


def test_route_special_values():
    """Large magnitudes, +-0 and saturated sigmoids stay exact."""
    E = 64
    logits = np.zeros((8, E), np.float32)
    logits[0] = np.linspace(-100, 100, E)
    logits[1, ::2] = -0.0
    logits[2] = 40.0   # sigmoid rounds to 1.0f everywhere: all keys tie
    logits[3] = -1e-30
    logits[4] = np.float32(3.4e38) * np.sign(np.arange(E) - 31.5)
    logits[5:] = np.random.default_rng(0).standard_normal((3, E)) * 30
    for method, ng, tg in [(0, 1, 1), (1, 1, 1), (4, 1, 1), (2, 8, 4), (2, 1, 1), (3, 1, 1),
                           (5, 1, 1), (6, 1, 1)]:
        w = wl.Workload("special", 97, T=8, H=128, E=E, I=128, k=8, method=method,
                        n_group=ng, topk_group=tg, bias=method in (2, 5))
        bias = torch.zeros(E) if method in (2, 5) else None
        check_route(w, torch.from_numpy(logits), bias)


# ------------------------------------------------------------------ permute
# Up to 8192 pairs the permute is one workgroup; above, three chunked
# kernels: both sides of the switch, and its edge, are covered.
@pytest.mark.parametrize("T,k,E,n_shared,dist", [
    (1, 1, 1, 0, "uniform"), (333, 2, 8, 0, "uniform"), (4096, 8, 256, 1, "uniform"),
    (8192, 8, 256, 1, "zipf"), (2048, 8, 128, 0, "one"), (1500, 3, 7, 2, "uniform"),
    (130, 8, 256, 0, "uniform"), (512, 8, 256, 0, "zipf"), (1024, 8, 64, 0, "one"),
    (8192, 1, 64, 0, "uniform"), (8193, 1, 64, 0, "uniform"), (9000, 8, 256, 1, "zipf"),
])
def test_permute_parity(T, k, E, n_shared, dist):
    rng = np.random.default_rng(T + k + E)
    if dist == "uniform":
        ids = rng.integers(0, E, size=(T, k))
    elif dist == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        ids = rng.choice(E, size=(T, k), p=p / p.sum())
    else:
        ids = np.full((T, k), E // 3)
    check_permute(ids.astype(np.int32), E, n_shared)


@pytest.mark.parametrize("T,k,E", [(300, 4, 64), (2000, 8, 256)])
def test_permute_clamps_out_of_range_ids(T, k, E):
    """Ids outside [0, E) are clamped into range (the boundary's reading of
    such input): the result is the stable sort of the clipped ids.  One case
    on each side of the one-workgroup switch (1200 and 16000 pairs)."""
    rng = np.random.default_rng(T * k)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.05
    ids[bad] = rng.choice(np.array([-1, -1000, E, E + 7, 2**31 - 1], np.int64), size=int(bad.sum())).astype(np.int32)
    off_g, pp_g, up_g = moe.permute(torch.from_numpy(ids).to(DEV), E, 0)
    off_o, pp_o, up_o = oracle.permute(np.clip(ids, 0, E - 1).astype(np.int32), E, 0)
    assert np.array_equal(host(off_g).numpy(), off_o)
    assert np.array_equal(host(pp_g).numpy(), pp_o)
    assert np.array_equal(host(up_g).numpy(), up_o)


# ------------------------------------------------------------ expert FFN
def small_workload(act, wdt, T=300, H=384, I=256, E=8, k=2, n_shared=0, method=4, **kw):
    return wl.Workload(f"small_{act}_{wdt}", 96, T=T, H=H, E=E, I=I, k=k, method=method,
                       act=act, wdt=wdt, n_shared=n_shared, **kw)


def run_ffn_check(w, inp, rows=None):
    """GPU expert_ffn fed the oracle's routing and permute; compare FFN rows."""
    ids, sc, _ = oracle_route(w, inp["logits"], inp["bias"])
    off, pp, up = oracle.permute(ids, w.E, w.n_shared)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    fc2 = moe.expert_ffn(g["x"], torch.from_numpy(off).to(DEV), torch.from_numpy(pp).to(DEV),
                         g["w13"], g["w2"], w.k, w.E, w.n_shared, g["w13_scale"], g["w2_scale"])
    if rows is None:
        rows = np.arange(w.R, dtype=np.int32)
    W = oracle.Weights(inp["w13"], inp["w2"], w.wdt, inp["w13_scale"], inp["w2_scale"])
    ref = oracle.expert_rows(W, inp["x"], w.act, w.T, w.k, w.E, w.n_shared, off, pp, rows)
    got = host(fc2).double().numpy()[rows]
    return rel_l2(got, ref), got, ref


@pytest.mark.parametrize("act,wdt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8")])
@pytest.mark.parametrize("shape", ["skinny", "wide"])
def test_expert_ffn_parity_small(act, wdt, shape):
    # skinny: ~19 rows per group (32-row tiles); wide: ~150 rows (128-row tiles),
    # ragged tails in both, several N- and K-tiles, one shared group.
    T = 300 if shape == "skinny" else 1200
    w = small_workload(act, wdt, T=T, E=32 if shape == "skinny" else 16, k=2, n_shared=1)
    inp = wl.make_inputs(w, 1)
    err, got, ref = run_ffn_check(w, inp)
    tol = TOL[(act, wdt)]
    # per-row relative errors too, so one bad tile cannot hide in the total
    row_err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert err < tol and row_err.max() < 3 * tol, (err, row_err.max())


def test_expert_ffn_empty_groups_and_one_hot():
    """Most experts empty, one expert holding every row, k = E = 1 degenerate."""
    w = small_workload("bf16", "bf16", T=257, E=16, k=1, method=0)
    inp = wl.make_inputs(w, 2)
    inp["logits"] = torch.full((w.T, w.E), -5.0)
    inp["logits"][:, 11] = 5.0
    err, _, _ = run_ffn_check(w, inp)
    assert err < 1e-2
    w1 = small_workload("f32", "f32", T=33, E=1, k=1, method=1)
    err1, _, _ = run_ffn_check(w1, wl.make_inputs(w1, 3))
    assert err1 < 1e-5


# group sizes on both sides of every tile-shape and row-class boundary
# (32/128/256-row tiles; classes [0,64), [64,384), [384,inf)) and of the
# remainder hand-off (513, 640: a big group's last <= 128 rows go to the mid
# launch; 641 keeps its 129-row remainder)
CLASS_EDGE_ROWS = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 160, 161, 255, 256, 257, 383, 384, 385, 511,
                   512, 513, 640, 641]


def edge_rows(counts, tail=40):
    """Rows of the permuted layout near every group's start and end (where
    tiles of different classes meet), for shapes too large to check in full."""
    off = np.concatenate([[0], np.cumsum(counts)])
    rows = set()
    for g in range(len(counts)):
        rows.update(range(off[g], min(off[g] + tail, off[g + 1])))
        rows.update(range(max(off[g + 1] - tail, off[g]), off[g + 1]))
    return np.array(sorted(rows), np.int32)


# H, I: K of FC1 / FC2.  Remainder hand-off between classes runs for K >= 4096,
# so (4096, 256) exercises it in FC1 and (256, 4096) in FC2.
@pytest.mark.parametrize("act,wdt,H,I", [("bf16", "bf16", 256, 256), ("bf16", "fp8", 256, 256),
                                         ("f32", "f32", 256, 256), ("bf16", "bf16", 4096, 256),
                                         ("bf16", "bf16", 256, 4096), ("bf16", "fp8", 4096, 256),
                                         ("bf16", "fp8", 256, 4096)])
def test_expert_ffn_row_class_boundaries(act, wdt, H, I):
    counts = CLASS_EDGE_ROWS
    E = len(counts)
    T = sum(counts)
    w = small_workload(act, wdt, T=T, H=H, I=I, E=E, k=1, method=0)
    inp = wl.make_inputs(w, 4)
    # top-1 routing that gives expert e exactly counts[e] tokens, in shuffled token order
    owner = np.repeat(np.arange(E), counts)
    np.random.default_rng(4).shuffle(owner)
    logits = torch.full((T, E), -5.0)
    logits[torch.arange(T), torch.from_numpy(owner)] = 5.0
    inp["logits"] = logits
    rows = None if H * I <= 256 * 256 else edge_rows(counts)
    err, got, ref = run_ffn_check(w, inp, rows)
    tol = TOL[(act, wdt)]
    row_err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert err < tol and row_err.max() < 3 * tol, (err, row_err.max())


def test_finalize_parity():
    """Finalize fed the oracle's FFN rows (rounded to bf16 / fp32)."""
    rng = np.random.default_rng(5)
    for T, k, H, n_shared, dt in [(77, 8, 7168, 1, torch.bfloat16), (64, 2, 256, 0, torch.float32),
                                  (300, 3, 1024, 2, torch.bfloat16)]:
        P = T * k
        rows = torch.from_numpy(rng.standard_normal((P + n_shared * T, H))).to(dt)
        ids = rng.integers(0, 16, size=(T, k)).astype(np.int32)
        _, _, up = oracle.permute(ids, 16, n_shared)
        sc = rng.random((T, k)).astype(np.float32)
        y = moe.finalize(rows.to(DEV), torch.from_numpy(up).to(DEV),
                         torch.from_numpy(sc).to(DEV), n_shared, out_dtype=torch.float32)
        ref = oracle.finalize(rows, "bf16" if dt == torch.bfloat16 else "f32", up,
                              sc.astype(np.float64), T, k, H, n_shared)
        assert rel_l2(host(y).numpy(), ref) < 1e-6


# ------------------------------------------------------------ whole layer
def sample_tokens(w, ids, n=16, seed=0):
    """First, last, random tokens, and tokens routed to the fullest / emptiest experts."""
    rng = np.random.default_rng(seed)
    cnt = np.bincount(ids.ravel(), minlength=w.E)
    pick = {0, w.T - 1, *rng.choice(w.T, size=min(n, w.T), replace=False).tolist()}
    for e in (int(np.argmax(cnt)), int(np.argmin(np.where(cnt > 0, cnt, 1 << 30)))):
        pick.add(int(np.nonzero(np.any(ids == e, 1))[0][0]))
    return np.array(sorted(pick), np.int32)


def run_layer(w, inp_dev):
    layer = moe.layer_for_workload(w, DEV)
    y = layer(inp_dev["x"], inp_dev["logits"], inp_dev["w13"], inp_dev["w2"], inp_dev["bias"],
              inp_dev["w13_scale"], inp_dev["w2_scale"])
    torch.cuda.synchronize()
    return layer, y


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_layer_parity_workloads(name):
    """Full-size layer on each workload: routing and permute compared in full,
    the layer output on sampled tokens (all tokens for the tiny workload)."""
    w = wl.WORKLOADS[name]
    print(f"[layer parity] {name} T={w.T} H={w.H} E={w.E} I={w.I} k={w.k}", flush=True)
    x = wl.make_x(w)
    logits = wl.make_logits(w, x)
    bias = wl.make_bias(w)
    w13, w2, s13, s2 = wl.make_weights(w, 0, DEV)
    g = dict(x=x.to(DEV), logits=logits.to(DEV), bias=None if bias is None else bias.to(DEV),
             w13=w13, w2=w2, w13_scale=s13, w2_scale=s2)
    layer, y = run_layer(w, g)
    ids, sc, hard = oracle_route(w, logits, bias)
    assert hard == 0
    assert np.array_equal(host(layer.ids).numpy(), ids)
    sc_g = host(layer.scales).numpy().astype(np.float64)
    assert np.max(np.abs(sc_g - sc) / np.abs(sc)) <= 1e-6
    off, pp, up = oracle.permute(ids, w.E, w.n_shared)
    assert np.array_equal(host(layer.offsets).numpy(), off)
    assert np.array_equal(host(layer.permuted_pair).numpy(), pp)
    assert np.array_equal(host(layer.unpermute).numpy(), up)
    toks = np.arange(w.T, dtype=np.int32) if w.T <= 64 else sample_tokens(w, ids)
    W = oracle.Weights(host(w13), host(w2), w.wdt, None if s13 is None else host(s13),
                       None if s2 is None else host(s2))
    ref = oracle.layer_tokens(W, x, w.act, w.T, w.k, w.E, w.n_shared, ids, sc, toks)
    got = host(y).double().numpy()[toks]
    err = rel_l2(got, ref)
    print(f"[layer parity] {name}: rel L2 {err:.3e} over {len(toks)} tokens", flush=True)
    assert err < TOL[(w.act, w.wdt)]
    assert not torch.isnan(y).any()


@pytest.mark.parametrize("wdt", ["bf16", "fp8"])
def test_layer_several_shared_experts(wdt):
    """Three shared experts (groups E, E+1, E+2: every token, weight 1) beside
    top-3 routed experts, whole layer against the oracle on every token."""
    w = small_workload("bf16", wdt, T=190, E=12, k=3, n_shared=3, method=1)
    inp = wl.make_inputs(w, 7)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    layer, y = run_layer(w, g)
    ids, sc, _ = oracle_route(w, inp["logits"], inp["bias"])
    W = oracle.Weights(inp["w13"], inp["w2"], wdt, inp["w13_scale"], inp["w2_scale"])
    toks = np.arange(w.T, dtype=np.int32)
    ref = oracle.layer_tokens(W, inp["x"], "bf16", w.T, w.k, w.E, w.n_shared, ids, sc, toks)
    assert rel_l2(host(y).double().numpy(), ref) < TOL[("bf16", wdt)]


def test_layer_nan_poisoned_buffers_and_determinism():
    """Outputs and workspace pre-filled with NaN must not leak; two runs agree bitwise."""
    w = small_workload("bf16", "bf16", T=500, E=16, k=4, n_shared=1, method=2, n_group=4,
                       topk_group=2, scaling=2.5, bias=True)
    inp = wl.make_inputs(w, 4)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    layer = moe.layer_for_workload(w, DEV)
    outs = []
    for _ in range(2):
        for buf in (layer.fc2_out, layer.y):
            buf.fill_(float("nan"))
        layer.ws.view(torch.uint8).fill_(0xFF)  # NaN patterns in bf16 / fp32
        y = layer(g["x"], g["logits"], g["w13"], g["w2"], g["bias"])
        torch.cuda.synchronize()
        assert not torch.isnan(y).any()
        outs.append(y.clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ids, sc, _ = oracle_route(w, inp["logits"], inp["bias"])
    W = oracle.Weights(inp["w13"], inp["w2"], "bf16")
    toks = np.arange(w.T, dtype=np.int32)
    ref = oracle.layer_tokens(W, inp["x"], "bf16", w.T, w.k, w.E, 1, ids, sc, toks)
    assert rel_l2(host(outs[0]).double().numpy(), ref) < 1e-2


@pytest.mark.parametrize("wdt", ["bf16", "fp8"])
def test_layer_graph_capture_replays(wdt):
    """The four calls captured into one HIP graph (no allocation, no host
    readback, no memset inside) replay to the eager result, bit for bit, also
    after the captured input buffers are refilled between replays."""
    w = small_workload("bf16", wdt, T=700, E=16, k=4, n_shared=1, method=2, n_group=4,
                       topk_group=2, scaling=2.5, bias=True)
    layer = moe.layer_for_workload(w, DEV)
    inputs = [{k: (None if v is None else v.to(DEV)) for k, v in wl.make_inputs(w, s).items()}
              for s in (11, 12)]
    g = {k: (None if v is None else v.clone()) for k, v in inputs[0].items()}  # captured buffers
    fwd = lambda: layer(g["x"], g["logits"], g["w13"], g["w2"], g["bias"],  # noqa: E731
                        g["w13_scale"], g["w2_scale"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y_graph = fwd()
    torch.cuda.synchronize()
    for rep in range(4):
        src = inputs[rep % 2]
        for k, v in src.items():
            if v is not None:
                g[k].copy_(v)
        torch.cuda.synchronize()
        eager = layer(src["x"], src["logits"], src["w13"], src["w2"], src["bias"],
                      src["w13_scale"], src["w2_scale"]).clone()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int16), eager.view(torch.int16)), rep
    ids, sc, _ = oracle_route(w, host(inputs[1]["logits"]), host(inputs[1]["bias"]))
    W = oracle.Weights(host(g["w13"]), host(g["w2"]), wdt,
                       None if g["w13_scale"] is None else host(g["w13_scale"]),
                       None if g["w2_scale"] is None else host(g["w2_scale"]))
    toks = np.arange(0, w.T, 7, dtype=np.int32)
    ref = oracle.layer_tokens(W, host(inputs[1]["x"]), "bf16", w.T, w.k, w.E, 1, ids, sc, toks)
    assert rel_l2(host(y_graph).double().numpy()[toks], ref) < TOL[("bf16", wdt)]


def test_zero_tokens_is_noop():
    w = small_workload("bf16", "bf16", T=0, E=8, k=2)
    L = moe.lib()
    assert L.moe_route(None, 0, 8, 0, 2, 1, 1, None, 1.0, 0, None, None, None) == 0
    assert L.moe_permute(None, 0, 2, 8, 0, None, None, None, None, 0, None) == 0
    assert L.moe_finalize(None, 1, None, None, 0, 2, 128, 0, None, 1, None) == 0
    assert L.moe_expert_ffn(None, 1, 0, 128, 128, 2, 8, 0, None, None, None, None, 1, None,
                            None, None, None, 0, None) == 0
    del w


def test_kernel_timing_hooks():
    w = small_workload("bf16", "bf16", T=256, E=8, k=2)
    inp = wl.make_inputs(w, 6)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    layer = moe.layer_for_workload(w, DEV)
    moe.timing_enable(True)
    try:
        moe.kernel_times(reset=True)
        for _ in range(3):
            layer(g["x"], g["logits"], g["w13"], g["w2"])
        t = moe.kernel_times(reset=True)
    finally:
        moe.timing_enable(False)
    # 512 pairs: the one-workgroup permute, not the chunked kernels
    for name in ("route", "permute_one", "finalize"):
        assert t[name][1] == 3 and t[name][0] > 0, (name, t[name])
    for name in ("permute_count", "permute_scan", "permute_scatter"):
        assert t[name][1] == 0, (name, t[name])
    # each grouped GEMM is one launch per row class (same count every call)
    for name in ("fc1", "fc2"):
        assert t[name][1] >= 3 and t[name][1] % 3 == 0 and t[name][0] > 0, (name, t[name])


def test_kernel_timing_collected_while_launching():
    """Reading and resetting the kernel times from one thread while another
    launches timed calls: every launch is counted exactly once, each with
    both of its events recorded."""
    import threading
    logits = torch.randn(512, 64, generator=torch.Generator().manual_seed(7)).to(DEV)
    n_calls, totals, errors = 400, [0], []
    done = threading.Event()

    def collect():
        try:
            while not done.is_set():
                totals[0] += moe.kernel_times(reset=True)["route"][1]
        except Exception as exc:  # reported by the main thread
            errors.append(exc)

    moe.timing_enable(True)
    try:
        moe.kernel_times(reset=True)
        reader = threading.Thread(target=collect)
        reader.start()
        for _ in range(n_calls):
            moe.route(logits, 4, 0)
        torch.cuda.synchronize()
        done.set()
        reader.join()
        last = moe.kernel_times(reset=True)["route"]
    finally:
        moe.timing_enable(False)
    assert not errors, errors
    assert totals[0] + last[1] == n_calls


def test_shared_expert_as_separate_call_on_second_stream():
    """The shared expert run as its own expert_ffn call (one group over all
    tokens, identity rows, writing fc2_out rows P..P+T) on a second stream,
    concurrent with route / permute / the routed FFN, gives the one-call
    layer's output bit for bit."""
    w = small_workload("bf16", "bf16", T=600, E=16, k=4, n_shared=1, method=2, n_group=4,
                       topk_group=2, scaling=2.5, bias=True)
    g = {k: (None if v is None else v.to(DEV)) for k, v in wl.make_inputs(w, 9).items()}
    layer = moe.layer_for_workload(w, DEV)
    y_one = layer(g["x"], g["logits"], g["w13"], g["w2"], g["bias"], None, None).clone()
    T, k, E, H, I, P = w.T, w.k, w.E, w.H, w.I, w.P
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    sc = torch.empty((T, k), dtype=torch.float32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    pp = torch.empty(P, dtype=torch.int32, device=DEV)
    up = torch.empty(P, dtype=torch.int32, device=DEV)
    fc2 = torch.full((P + T, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws_r = moe.alloc_workspace(T, k, E, 0, H, I, torch.bfloat16, DEV)
    ws_s = moe.alloc_workspace(T, 1, 1, 0, H, I, torch.bfloat16, DEV)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        moe.expert_ffn(g["x"], torch.tensor([0, T], dtype=torch.int32, device=DEV),
                       torch.arange(T, dtype=torch.int32, device=DEV), g["w13"][E:E + 1],
                       g["w2"][E:E + 1], 1, 1, 0, ws=ws_s, out=fc2[P:])
    moe.route(g["logits"], k, w.method, w.n_group, w.topk_group, g["bias"], w.scaling, False,
              out=(ids, sc))
    moe.permute(ids, E, 0, ws=ws_r, out=(off, pp, up))
    moe.expert_ffn(g["x"], off, pp, g["w13"][:E], g["w2"][:E], k, E, 0, ws=ws_r, out=fc2[:P])
    main.wait_stream(side)
    y_split = moe.finalize(fc2, up, sc, 1)
    torch.cuda.synchronize()
    assert torch.equal(y_split.view(torch.int16), y_one.view(torch.int16))
