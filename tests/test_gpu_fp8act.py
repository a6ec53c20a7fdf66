"""GPU parity of the fp8-activation path (moe_quantize_fp8 + moe_expert_ffn_fp8)
against the CPU oracle, through the C ABI.

Bars: codes and scales of the 1x128 quantiser bit-exact; FFN rows and layer
output within relative L2 1e-2 (per row 5e-2); the quantised h in the
workspace: scales within 1e-3 relative, every code a correct rounding of the
oracle's h up to 1e-3 of its block maximum (one fp8 MFMA sums its 128
products with ~13-bit precision).  The oracle quantises x the
same way (bit-exact, checked first) and quantises its fp64 h rounded to fp32;
the GPU quantises its fp32-accumulated h, so the codes of h differ only where
an fp32 rounding difference crosses an e4m3 rounding midpoint (rare), and the
remaining difference is the bf16 rounding of fc2_out and y (~2e-3 each).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import mixture_experts_layer_07_amd as moe
from mixture_experts_layer_07_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 1e-2
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_quant_handworked.json")


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def host(t):
    return t.detach().cpu()


def gpu_quantize(x):
    xq, xs = moe.quantize_fp8(x.to(DEV))
    return host(xq).view(torch.uint8).numpy(), host(xs).numpy()


def oracle_quantize(x):
    if x.dtype == torch.bfloat16:
        return oracle.quantize_fp8(x.view(torch.int16).numpy(), "bf16")
    return oracle.quantize_fp8(x.numpy(), "f32")


def blocky(rng, rows, cols, lo=-30, hi=30, dtype=torch.bfloat16):
    """Rows whose 128-value blocks span many magnitudes, with zero blocks and -0."""
    mag = np.exp2(rng.integers(lo, hi, (rows, cols // 128, 1)).astype(np.float64))
    x = (rng.standard_normal((rows, cols // 128, 128)) * mag).reshape(rows, cols)
    x[rng.random((rows, cols)) < 0.01] = -0.0
    zero = rng.random((rows, cols // 128)) < 0.05
    x.reshape(rows, cols // 128, 128)[zero] = 0.0
    return torch.from_numpy(x).to(dtype)


@pytest.mark.parametrize("rows,cols,dtype", [(1, 128, torch.bfloat16), (7, 384, torch.bfloat16),
                                             (333, 7168, torch.bfloat16), (64, 4096, torch.float32),
                                             (1000, 256, torch.float32)])
def test_quantize_fp8_bit_exact(rows, cols, dtype):
    x = blocky(np.random.default_rng(rows + cols), rows, cols, dtype=dtype)
    qg, sg = gpu_quantize(x)
    qo, so = oracle_quantize(x)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32)), "scales differ"
    assert np.array_equal(qg, qo), f"{np.sum(qg != qo)} codes differ"


def test_quantize_fp8_tiny_and_subnormal_blocks():
    """Blocks whose values (and scale) are fp32 subnormal, and a block whose
    scale underflows to 0 (encodes as zeros)."""
    x = np.zeros((4, 256), np.float32)
    x[0, :128] = np.float32(1e-39) * np.arange(1, 129, dtype=np.float32) / 128
    x[1, :128] = np.linspace(-3e-38, 3e-38, 128, dtype=np.float32)
    x[2, 5] = np.float32(1e-44)                      # amax / 448 underflows: s = 0
    x[3, 128:] = np.float32(2.0 ** -126) * np.linspace(-1, 1, 128, dtype=np.float32)
    xt = torch.from_numpy(x)
    qg, sg = gpu_quantize(xt)
    qo, so = oracle_quantize(xt)
    assert so[2, 0] == 0 and np.all(qo[2] == 0)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo)


def test_quantize_fp8_handworked_golden():
    doc = json.load(open(GOLDEN))
    for case in doc["cases"]:
        x = torch.tensor(case["x"], dtype=torch.float32)
        qg, sg = gpu_quantize(x)
        head = np.array(case["codes_head"], np.uint8)
        n = head.shape[1]
        assert np.array_equal(qg[:, :n], head), case["name"]
        assert np.all(qg[:, n:] == 0), case["name"]
        assert np.array_equal(sg, np.array(case["scales"], np.float32)), case["name"]


def test_quantize_fp8_zero_rows_and_errors():
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    xq, xs = moe.quantize_fp8(x)
    assert xq.shape == (0, 256) and xs.shape == (0, 2)
    with pytest.raises(moe.MoeError):
        moe.quantize_fp8(torch.zeros((4, 200), dtype=torch.bfloat16, device=DEV))


# ------------------------------------------------------------ expert FFN
def fp8_workload(T, H, I, E, k, n_shared=0, method=4, **kw):
    return wl.Workload(f"fp8act_{T}_{E}", 97, T=T, H=H, E=E, I=I, k=k, method=method,
                       act="bf16", wdt="fp8", n_shared=n_shared, **kw)


def check_h_codes(w, ws, h_ref):
    """The quantised intermediate left in the workspace (hq [R, I] e4m3 at 0,
    its scales [R, I/128] at the next 256-byte boundary) against the oracle's
    fp64 h.  One fp8 MFMA sums its 128 products with ~13-bit precision
    (measured on MI355X: error up to 1.7e-4 of the sum of |products|), and
    the GPU adds one such sum per 128-wide K block, so its h (and the block
    maximum) can differ from the oracle's by ~1e-4 relative: the scales must
    match within 1e-3, and every GPU code must be a round-to-nearest e4m3
    code of a value within 1e-3 of the block maximum of the oracle's h.
    Returns the fraction of codes that differ from the oracle's own
    quantisation."""
    R, I = w.R, w.I
    hq = host(ws[:R * I]).numpy().reshape(R, I)
    off = (R * I + 255) // 256 * 256
    hs = host(ws[off:off + R * (I // 128) * 4]).numpy().view(np.float32).reshape(R, I // 128)
    qo, so = oracle.quantize_fp8(h_ref.astype(np.float32), "f32")
    rel = np.abs(hs.astype(np.float64) - so) / np.maximum(so, 1e-30)
    assert rel.max() < 1e-3, f"h scale rel diff {rel.max()}"
    table = np.array([oracle.decode_e4m3(c) for c in range(256)])
    s_g = np.repeat(hs.astype(np.float64), 128, axis=1)
    v = table[hq] * s_g
    amax = np.repeat(np.abs(h_ref).reshape(R, I // 128, 128).max(axis=2), 128, axis=1)
    m = np.maximum(np.abs(v), np.abs(h_ref)) / np.maximum(s_g, 1e-300)
    step = np.where(m >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(m, 2.0 ** -6))) - 3), 2.0 ** -9)
    err = np.abs(v - h_ref)
    allowed = step / 2 * s_g * (1 + 1e-6) + 1e-3 * amax
    bad = err > allowed
    assert not bad.any(), f"{int(bad.sum())} h codes off by more than rounding + 1e-3 of the block max"
    return float((hq != qo).mean())


def run_ffn_fp8_check(w, inp, rows=None):
    """GPU quantize + expert_ffn_fp8 fed the oracle's routing and permute."""
    ids, sc, _ = oracle.route(inp["logits"], w.k, w.method, w.n_group, w.topk_group, inp["bias"],
                              w.scaling, bool(w.flags & wl.ROUTE_FLAG_RENORMALIZE))
    off, pp, up = oracle.permute(ids, w.E, w.n_shared)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    xq, xs = moe.quantize_fp8(g["x"])
    qo, so = oracle_quantize(inp["x"])
    assert np.array_equal(host(xq).view(torch.uint8).numpy(), qo)
    assert np.array_equal(host(xs).numpy(), so)
    ws = moe.alloc_workspace(w.T, w.k, w.E, w.n_shared, w.H, w.I, torch.float8_e4m3fn, DEV)
    fc2 = moe.expert_ffn_fp8(xq, xs, torch.from_numpy(off).to(DEV), torch.from_numpy(pp).to(DEV),
                             g["w13"], g["w2"], g["w13_scale"], g["w2_scale"], w.k, w.E, w.n_shared,
                             ws=ws)
    all_rows = rows is None
    if all_rows:
        rows = np.arange(w.R, dtype=np.int32)
    W = oracle.Weights(inp["w13"], inp["w2"], "fp8", inp["w13_scale"], inp["w2_scale"])
    ref, h = oracle.expert_rows(W, qo, "fp8", w.T, w.k, w.E, w.n_shared, off, pp, rows, want_h=True,
                                x_scale=so)
    if all_rows:
        frac = check_h_codes(w, ws, h)
        print(f"[fp8 ffn] {frac:.2e} of h codes differ from the oracle's", flush=True)
        assert frac < 1e-2
    got = host(fc2).double().numpy()[rows]
    return rel_l2(got, ref), got, ref


# A single h code one step off moves a row by about 6% of that element's share
# of the row (|h_i| / ||h||), so the per-row bar is wider than the total one.
ROW_TOL = 5e-2


@pytest.mark.parametrize("shape", ["skinny", "wide"])
def test_expert_ffn_fp8_parity_small(shape):
    # skinny: ~19 rows per group (32-row tiles); wide: ~150 rows (128-row tiles),
    # ragged tails, several N- and K-tiles, one shared group (256-row tiles).
    T = 300 if shape == "skinny" else 1200
    w = fp8_workload(T, 384, 256, 32 if shape == "skinny" else 16, 2, n_shared=1)
    err, got, ref = run_ffn_fp8_check(w, wl.make_inputs(w, 1))
    row_err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    print(f"[fp8 ffn {shape}] rel L2 {err:.3e}, worst row {row_err.max():.3e}", flush=True)
    assert err < TOL and row_err.max() < ROW_TOL, (err, row_err.max())


CLASS_EDGE_ROWS = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 160, 161, 255, 256, 257, 383, 384, 385, 511,
                   512, 513, 640, 641]


@pytest.mark.parametrize("H,I", [(256, 384), (4096, 256), (256, 4096)])
def test_expert_ffn_fp8_row_class_boundaries(H, I):
    # (4096, 256) / (256, 4096): FC1 / FC2 with K >= 4096, where a group's last
    # partial tile is handed to the next smaller tile shape
    counts = CLASS_EDGE_ROWS
    E = len(counts)
    T = sum(counts)
    w = fp8_workload(T, H, I, E, 1, method=0)
    inp = wl.make_inputs(w, 4)
    owner = np.repeat(np.arange(E), counts)
    np.random.default_rng(4).shuffle(owner)
    logits = torch.full((T, E), -5.0)
    logits[torch.arange(T), torch.from_numpy(owner)] = 5.0
    inp["logits"] = logits
    rows = None
    if H * I > 256 * 384:
        off = np.concatenate([[0], np.cumsum(counts)])
        sel = set()
        for g in range(E):
            sel.update(range(off[g], min(off[g] + 40, off[g + 1])))
            sel.update(range(max(off[g + 1] - 40, off[g]), off[g + 1]))
        rows = np.array(sorted(sel), np.int32)
    err, got, ref = run_ffn_fp8_check(w, inp, rows)
    row_err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert err < TOL and row_err.max() < ROW_TOL, (err, row_err.max())


def test_expert_ffn_fp8_empty_groups_one_hot():
    w = fp8_workload(257, 256, 256, 16, 1, method=0)
    inp = wl.make_inputs(w, 2)
    inp["logits"] = torch.full((w.T, w.E), -5.0)
    inp["logits"][:, 11] = 5.0
    err, _, _ = run_ffn_fp8_check(w, inp)
    assert err < TOL


def test_expert_ffn_fp8_rejects_bad_shapes():
    w = fp8_workload(16, 256, 256, 4, 2)
    inp = {k: (None if v is None else v.to(DEV)) for k, v in wl.make_inputs(w, 3).items()}
    xq, xs = moe.quantize_fp8(inp["x"])
    off = torch.zeros(w.E + 1, dtype=torch.int32, device=DEV)
    pp = torch.zeros(w.P, dtype=torch.int32, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.expert_ffn_fp8(xq, xs, off, pp, inp["w13"], inp["w2"], inp["w13_scale"], inp["w2_scale"],
                           w.k, w.E, ws=ws)
    assert e.value.status == 3  # MOE_ERR_WORKSPACE


# ------------------------------------------------------------ whole layer
def sample_tokens(T, ids, E, n=16, seed=0):
    rng = np.random.default_rng(seed)
    cnt = np.bincount(ids.ravel(), minlength=E)
    pick = {0, T - 1, *rng.choice(T, size=min(n, T), replace=False).tolist()}
    for e in (int(np.argmax(cnt)), int(np.argmin(np.where(cnt > 0, cnt, 1 << 30)))):
        pick.add(int(np.nonzero(np.any(ids == e, 1))[0][0]))
    return np.array(sorted(pick), np.int32)


FP8ACT_WORKLOADS = {"qwen3_fp8": wl.WORKLOADS["qwen3_fp8"], **wl.FP8_WORKLOADS}


@pytest.mark.parametrize("name", list(FP8ACT_WORKLOADS))
def test_layer_fp8act_workloads(name):
    """Full-size layer with fp8 activations: sampled tokens against the oracle."""
    w = FP8ACT_WORKLOADS[name]
    print(f"[fp8act layer] {name} T={w.T} H={w.H} E={w.E} I={w.I} k={w.k}", flush=True)
    x = wl.make_x(w)
    logits = wl.make_logits(w, x)
    bias = wl.make_bias(w)
    w13, w2, s13, s2 = wl.make_weights(w, 0, DEV)
    layer = moe.layer_for_workload(w, DEV, fp8_act=True)
    y = layer(x.to(DEV), logits.to(DEV), w13, w2, None if bias is None else bias.to(DEV), s13, s2)
    torch.cuda.synchronize()
    ids, sc, hard = oracle.route(logits, w.k, w.method, w.n_group, w.topk_group, bias, w.scaling,
                                 bool(w.flags & wl.ROUTE_FLAG_RENORMALIZE))
    assert hard == 0
    assert np.array_equal(host(layer.ids).numpy(), ids)
    qo, so = oracle_quantize(x)
    assert np.array_equal(host(layer.xq).view(torch.uint8).numpy(), qo)
    assert np.array_equal(host(layer.x_scale).numpy(), so)
    toks = sample_tokens(w.T, ids, w.E)
    W = oracle.Weights(host(w13), host(w2), "fp8", host(s13), host(s2))
    ref = oracle.layer_tokens(W, qo, "fp8", w.T, w.k, w.E, w.n_shared, ids, sc, toks, x_scale=so)
    got = host(y).double().numpy()[toks]
    err = rel_l2(got, ref)
    print(f"[fp8act layer] {name}: rel L2 {err:.3e} over {len(toks)} tokens", flush=True)
    assert err < TOL
    assert not torch.isnan(y).any()


def test_layer_fp8act_determinism_and_nan_poison():
    w = fp8_workload(500, 256, 256, 16, 4, n_shared=1, method=2, n_group=4, topk_group=2,
                     scaling=2.5, bias=True)
    inp = {k: (None if v is None else v.to(DEV)) for k, v in wl.make_inputs(w, 4).items()}
    layer = moe.layer_for_workload(w, DEV, fp8_act=True)
    outs = []
    for _ in range(2):
        layer.ws.fill_(0xFF)  # NaN in every fp32 / e4m3 / bf16 view
        layer.fc2_out.fill_(float("nan"))
        layer.y.fill_(float("nan"))
        y = layer(inp["x"], inp["logits"], inp["w13"], inp["w2"], inp["bias"], inp["w13_scale"],
                  inp["w2_scale"])
        torch.cuda.synchronize()
        assert not torch.isnan(y).any()
        outs.append(y.clone())
    assert torch.equal(outs[0], outs[1])


def test_layer_fp8act_graph_capture_replays():
    """route, permute, quantize_fp8, expert_ffn_fp8 and finalize captured into
    one HIP graph replay to the eager result bit for bit, also after the
    captured input buffers are refilled between replays."""
    w = fp8_workload(700, 256, 256, 16, 4, n_shared=1, method=2, n_group=4, topk_group=2,
                     scaling=2.5, bias=True)
    layer = moe.layer_for_workload(w, DEV, fp8_act=True)
    inputs = [{k: (None if v is None else v.to(DEV)) for k, v in wl.make_inputs(w, s).items()}
              for s in (11, 12)]
    g = {k: (None if v is None else v.clone()) for k, v in inputs[0].items()}
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
    x1 = host(inputs[1]["x"])
    ids, sc, _ = oracle.route(host(inputs[1]["logits"]), w.k, w.method, w.n_group, w.topk_group,
                              host(inputs[1]["bias"]), w.scaling, False)
    qo, so = oracle_quantize(x1)
    W = oracle.Weights(host(g["w13"]), host(g["w2"]), "fp8", host(g["w13_scale"]), host(g["w2_scale"]))
    toks = np.arange(0, w.T, 7, dtype=np.int32)
    ref = oracle.layer_tokens(W, qo, "fp8", w.T, w.k, w.E, 1, ids, sc, toks, x_scale=so)
    assert rel_l2(host(y_graph).double().numpy()[toks], ref) < TOL


@pytest.mark.parametrize("T,H,I,E,k,n_shared", [(1, 128, 128, 1, 1, 0), (3, 256, 128, 4, 4, 2),
                                                (17, 384, 640, 5, 2, 1)])
def test_expert_ffn_fp8_degenerate_shapes(T, H, I, E, k, n_shared):
    """One token and one expert; k = E with two shared experts; H and I that
    leave partial 256-wide N tiles in both GEMMs."""
    w = fp8_workload(T, H, I, E, k, n_shared=n_shared, method=4)
    err, got, ref = run_ffn_fp8_check(w, wl.make_inputs(w, 5))
    row_err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert err < TOL and row_err.max() < ROW_TOL, (err, row_err.max())
