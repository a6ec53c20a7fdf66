"""Whole groups at the production shape: every FFN row of selected groups of
the DeepSeek-V3-shaped prefill batch (T=8192, H=7168, I=2048, 256 experts +
1 shared, top-8, Zipf-skewed routing) against the oracle, on the two-call
path in bf16 and in fp8 x fp8.

The groups cover every tile class and edge of the grouped GEMMs at this
shape: the fullest expert (6809 rows: 26 full 256-row tiles and a 153-row
partial one), the smallest big group whose last partial tile goes to the
128-row tiles in FC1 (564 rows: two 256-row tiles and a 52-row tail), the
largest mid-class group (328 rows: 128-row tiles with a ragged tail) and the
largest skinny group (63 rows: 32-row tiles); row counts at seed 0.  The
routing and permute come from the oracle (they are compared in full by the
layer tests), so the GEMMs see exactly the oracle's rows.  Every row of each
group is compared: relative L2 over the group and per row.
"""
import numpy as np
import pytest
import torch

import oracle
import mixture_experts_layer_07_amd as moe
from mixture_experts_layer_07_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


def select_groups(counts):
    """(label, group) pairs: fullest, big with an FC1 hand-off tail, mid, skinny."""
    E = len(counts)
    fullest = int(np.argmax(counts))
    handoff = [g for g in range(E) if counts[g] >= 384 and 1 <= counts[g] % 256 <= 128]
    mid = [g for g in range(E) if 64 <= counts[g] < 384]
    skinny = [g for g in range(E) if 0 < counts[g] < 64]
    out = [("fullest", fullest)]
    if handoff:
        out.append(("big, FC1 hand-off tail", min(handoff, key=lambda g: counts[g])))
    if mid:
        out.append(("mid", max(mid, key=lambda g: counts[g])))
    if skinny:
        out.append(("skinny", max(skinny, key=lambda g: counts[g])))
    return out


def host_weights(w, dev_w13, dev_w2, s13, s2, groups):
    """oracle.Weights over full-size host arrays of which only `groups` are
    filled (the rest are never read: untouched host pages stay unallocated)."""
    h13 = torch.empty(dev_w13.shape, dtype=dev_w13.dtype)
    h2 = torch.empty(dev_w2.shape, dtype=dev_w2.dtype)
    for g in groups:
        h13[g] = dev_w13[g].cpu()
        h2[g] = dev_w2[g].cpu()
    return oracle.Weights(h13, h2, w.wdt, None if s13 is None else s13.cpu(),
                          None if s2 is None else s2.cpu())


def check_groups(w, fc2, W, x_host, act, off, pp, groups, x_scale=None, row_bar=3e-2):
    got_all = fc2.cpu()
    for label, g in groups:
        rows = np.arange(off[g], off[g + 1], dtype=np.int32)
        print(f"production groups {w.name}: {label} group {g}, {len(rows)} rows", flush=True)
        ref = oracle.expert_rows(W, x_host, act, w.T, w.k, w.E, w.n_shared, off, pp, rows,
                                 x_scale=x_scale)
        got = got_all[rows].double().numpy()
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        row_err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
        print(f"   rel L2 {err:.3e}, worst row {row_err.max():.3e}", flush=True)
        assert err < 1e-2, f"{label} group {g}: rel L2 {err}"
        assert row_err.max() < row_bar, f"{label} group {g}: row {int(row_err.argmax())} err {row_err.max()}"


@pytest.fixture(scope="module")
def prefill_routing():
    """x, offsets, permuted_pair and per-expert counts of the prefill batch (the
    bf16 and fp8-weight workloads share x, logits and bias)."""
    w = wl.WORKLOADS["dsv3_prefill"]
    x = wl.make_x(w)
    logits = wl.make_logits(w, x)
    bias = wl.make_bias(w)
    ids, _, hard = oracle.route(logits, w.k, w.method, w.n_group, w.topk_group, bias, w.scaling, False)
    assert hard == 0
    off, pp, _ = oracle.permute(ids, w.E, w.n_shared)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    return x, off, pp, counts


# the fullest group alone (the oracle needs about 90 s for its 6809 rows on 16 cores), then the others
PARTS = ["fullest", "others"]


def part_groups(counts, part):
    sel = select_groups(counts)
    return sel[:1] if part == "fullest" else sel[1:]


@pytest.mark.parametrize("part", PARTS)
def test_prefill_groups_bf16_every_row(prefill_routing, part):
    x, off, pp, counts = prefill_routing
    w = wl.WORKLOADS["dsv3_prefill"]
    groups = part_groups(counts, part)
    w13, w2, _, _ = wl.make_weights(w, 0, DEV)
    fc2 = moe.expert_ffn(x.to(DEV), torch.from_numpy(off).to(DEV), torch.from_numpy(pp).to(DEV),
                         w13, w2, w.k, w.E, w.n_shared)
    torch.cuda.synchronize()
    W = host_weights(w, w13, w2, None, None, [g for _, g in groups])
    del w13, w2
    torch.cuda.empty_cache()
    check_groups(w, fc2, W, x, w.act, off, pp, groups)


@pytest.mark.parametrize("part", PARTS)
def test_prefill_groups_fp8_activations_every_row(prefill_routing, part):
    x, off, pp, counts = prefill_routing
    w = wl.FP8_WORKLOADS["dsv3_prefill_fp8"]
    groups = part_groups(counts, part)
    w13, w2, s13, s2 = wl.make_weights(w, 0, DEV)
    xq, xs = moe.quantize_fp8(x.to(DEV))
    torch.cuda.synchronize()
    xq_o, xs_o = oracle.quantize_fp8(x.view(torch.int16).numpy(), "bf16")
    assert np.array_equal(xq.view(torch.uint8).cpu().numpy(), xq_o), "x codes differ from the oracle's"
    assert np.array_equal(xs.cpu().numpy(), xs_o), "x scales differ from the oracle's"
    fc2 = moe.expert_ffn_fp8(xq, xs, torch.from_numpy(off).to(DEV), torch.from_numpy(pp).to(DEV),
                             w13, w2, s13, s2, w.k, w.E, w.n_shared)
    torch.cuda.synchronize()
    W = host_weights(w, w13, w2, s13, s2, [g for _, g in groups])
    del w13, w2, s13, s2
    torch.cuda.empty_cache()
    check_groups(w, fc2, W, xq_o, "fp8", off, pp, groups, x_scale=xs_o, row_bar=5e-2)
