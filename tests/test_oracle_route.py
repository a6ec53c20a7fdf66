"""Pins of the oracle's routing (no GPU).

Routing methods follow the RoutingMethodType comments and the noaux_tc section
of "TensorRT-LLM 源码完全拆解(十三): MoE 层前向执行" and the FusedTopKRouter
section of "vLLM 源码完全拆解(八): MoE 层的前向执行".  Each check below computes
the expected value another way: exhaustive enumeration of index subsets,
decimal arithmetic at 60 digits, or torch library routines.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from pins import (brute_group_score, brute_topk, ordered_by_key, sigmoid_decimal,
                  sigmoid_f32_exact)

GRID = np.array([-2, -1, 0, 1, 2], np.float32) / np.float32(4)  # tie-heavy, exact in fp32


def tie_logits(rng, T, E):
    return rng.choice(GRID, size=(T, E)).astype(np.float32)


# ------------------------------------------------------------- softmax family
@pytest.mark.parametrize("E", [4, 6, 8, 12, 16])
def test_softmax_selection_brute_force(orc, E):
    rng = np.random.default_rng(100 + E)
    ks = range(1, E + 1) if E <= 12 else [1, 2, 3, 8, 15, 16]
    for k in ks:
        lg = tie_logits(rng, 3, E)
        for method, renorm in [(orc.DEFAULT, False), (orc.DEFAULT, True),
                               (orc.RENORMALIZE, False), (orc.RENORMALIZE_NAIVE, False)]:
            ids, sc, _ = orc.route(lg, k, method, renorm=renorm)
            for t in range(lg.shape[0]):
                keys = [float(v) for v in lg[t]]
                assert tuple(sorted(ids[t])) == brute_topk(keys, k), (E, k, t)
                assert ordered_by_key(list(ids[t]), keys)


def test_softmax_selection_random_continuous(orc):
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((20, 10)).astype(np.float32)
    ids, _, _ = orc.route(lg, 4, orc.RENORMALIZE_NAIVE)
    for t in range(20):
        assert tuple(sorted(ids[t])) == brute_topk([float(v) for v in lg[t]], 4)


def test_default_scales_are_torch_softmax(orc):
    """Default without renormalise: the selected softmax probabilities."""
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal((16, 12)) * 3).astype(np.float32)
    ids, sc, _ = orc.route(lg, 5, orc.DEFAULT)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=-1).numpy()
    np.testing.assert_allclose(sc, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13)
    # k = E: all probabilities, which sum to one
    ids, sc, _ = orc.route(lg, 12, orc.DEFAULT)
    np.testing.assert_allclose(sc.sum(1), 1.0, rtol=1e-13)


def test_renormalized_scales_closed_form(orc):
    """Renormalised softmax over S: scales sum to `scaling`, and the ratio of
    two scales is exp of the logit difference."""
    rng = np.random.default_rng(4)
    lg = (rng.standard_normal((16, 16)) * 2).astype(np.float32)
    for method, renorm in [(orc.DEFAULT, True), (orc.RENORMALIZE, False),
                           (orc.RENORMALIZE_NAIVE, False)]:
        ids, sc, _ = orc.route(lg, 6, method, renorm=renorm, scaling=1.75)
        np.testing.assert_allclose(sc.sum(1), 1.75, rtol=1e-13)
        sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), 1)
        np.testing.assert_allclose(sc[:, 1:] / sc[:, :1], np.exp(sel[:, 1:] - sel[:, :1]),
                                   rtol=1e-12)
        assert np.all(np.diff(sc, axis=1) <= 0)


def test_softmax_methods_equivalent(orc):
    """Default+renormalise == Renormalize == RenormalizeNaive in exact arithmetic."""
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((64, 32)).astype(np.float32)
    a = orc.route(lg, 8, orc.DEFAULT, renorm=True)
    b = orc.route(lg, 8, orc.RENORMALIZE)
    c = orc.route(lg, 8, orc.RENORMALIZE_NAIVE)
    assert np.array_equal(a[0], b[0]) and np.array_equal(b[0], c[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)
    np.testing.assert_allclose(b[1], c[1], rtol=1e-12)


# ---------------------------------------------------------------- DeepSeek-V3
def test_sigmoid_f32_matches_decimal(orc):
    rng = np.random.default_rng(6)
    vals = list(rng.standard_normal(3000).astype(np.float32) * np.float32(4))
    vals += [0.0, -0.0, 1e-30, -1e-30, 1e-8, 88.0, -88.0, 103.9, -103.9, 17.0, -17.0,
             float(np.float32(math.log(3.0)))]
    hard_total = 0
    for v in vals:
        got, hard = orc.sigmoid_f32(float(v))
        hard_total += hard
        assert np.float32(got) == sigmoid_f32_exact(float(np.float32(v))), v
    assert hard_total == 0


def dsv3_reference(lg, bias, k, n_group, topk_group, scaling):
    """Enumeration-based DeepSeek-V3 selection with decimal sigmoid."""
    T, E = lg.shape
    gsz = E // n_group
    out_ids, out_sc = [], []
    for t in range(T):
        sig = [sigmoid_f32_exact(float(v)) for v in lg[t]]
        kap = [np.float32(sig[e] + np.float32(bias[e])) for e in range(E)]
        gs = [brute_group_score(kap, range(g * gsz, (g + 1) * gsz)) for g in range(n_group)]
        gsel = brute_topk([float(v) for v in gs], topk_group)
        allowed = [(e // gsz) in gsel for e in range(E)]
        S = brute_topk([float(v) for v in kap], k, allowed)
        out_ids.append((S, kap))
        den = sum(float(sig[e]) for e in S) + 1e-20
        out_sc.append({e: float(sig[e]) / den * scaling for e in S})
    return out_ids, out_sc


@pytest.mark.parametrize("E,n_group", [(4, 2), (6, 3), (8, 1), (8, 2), (8, 4), (12, 3),
                                       (12, 6), (16, 4), (16, 8)])
def test_dsv3_brute_force(orc, E, n_group):
    rng = np.random.default_rng(1000 + E * 10 + n_group)
    gsz = E // n_group
    for topk_group in range(1, n_group + 1):
        for k in sorted({1, 2, min(3, topk_group * gsz), topk_group * gsz}):
            lg = tie_logits(rng, 2, E)
            bias = (rng.choice(GRID, size=E) / np.float32(2)).astype(np.float32)
            ids, sc, hard = orc.route(lg, k, orc.DEEPSEEKV3, n_group, topk_group, bias, 2.5)
            assert hard == 0
            ref_ids, ref_sc = dsv3_reference(lg, bias, k, n_group, topk_group, 2.5)
            for t in range(lg.shape[0]):
                S, kap = ref_ids[t]
                assert tuple(sorted(ids[t])) == S, (E, n_group, topk_group, k, t)
                assert ordered_by_key(list(ids[t]), [float(v) for v in kap])
                for j, e in enumerate(ids[t]):
                    assert sc[t, j] == pytest.approx(ref_sc[t][e], rel=1e-13)


def test_dsv3_group_step_noop_and_single_group(orc):
    """topk_group == n_group keeps every group, which is the same selection as
    one group; with one group the method is sigmoid + bias -> top-k ->
    unbiased renormalise (the MiniMax2 comment), and with zero bias it is
    sigmoid -> top-k -> renormalise (the SigmoidRenorm comment)."""
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((32, 64)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, 64).astype(np.float32)
    a = orc.route(lg, 8, orc.DEEPSEEKV3, 8, 8, bias, 1.0)
    b = orc.route(lg, 8, orc.DEEPSEEKV3, 1, 1, bias, 1.0)
    assert np.array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-15)
    for use_bias in (True, False):
        bb = bias if use_bias else np.zeros(64, np.float32)
        ids, sc, _ = orc.route(lg, 8, orc.DEEPSEEKV3, 1, 1, bb, 1.0)
        sig = np.array([[sigmoid_f32_exact(float(v)) for v in row] for row in lg], np.float32)
        kap = (sig + bb[None, :]).astype(np.float32)
        for t in range(32):
            order = np.lexsort((np.arange(64), -kap[t].astype(np.float64)))[:8]
            assert list(ids[t]) == list(order)
            w = sig[t, order].astype(np.float64)
            np.testing.assert_allclose(sc[t], w / (w.sum() + 1e-20), rtol=1e-13)


def test_dsv3_bias_only_selects(orc):
    """A large bias forces an expert in, yet its weight uses the unbiased score."""
    lg = np.zeros((1, 8), np.float32)
    lg[0, 3] = -4.0
    bias = np.zeros(8, np.float32)
    bias[3] = 1.0
    ids, sc, _ = orc.route(lg, 2, orc.DEEPSEEKV3, 1, 1, bias, 1.0)
    assert ids[0, 0] == 3 and ids[0, 1] == 0
    s3 = float(sigmoid_f32_exact(-4.0))
    np.testing.assert_allclose(sc[0], [s3 / (s3 + 0.5), 0.5 / (s3 + 0.5)], rtol=1e-13)


# ------------------------------------------- sigmoid family without grouping
def sigmoid_reference(lg, bias, k, scaling):
    """MiniMax2 / SigmoidRenorm by enumeration: decimal sigmoid rounded to fp32,
    optional bias added in fp32 for the key, unbiased sigmoids renormalised."""
    out = []
    for row in lg:
        sig = [sigmoid_f32_exact(float(v)) for v in row]
        kap = [np.float32(sig[e] + np.float32(bias[e])) if bias is not None else sig[e]
               for e in range(len(row))]
        S = brute_topk([float(v) for v in kap], k)
        den = sum(float(sig[e]) for e in S)
        out.append((S, kap, {e: float(sig[e]) / den * scaling for e in S}))
    return out


@pytest.mark.parametrize("E", [4, 6, 8, 12])
@pytest.mark.parametrize("use_bias", [True, False])
def test_sigmoid_methods_brute_force(orc, E, use_bias):
    """MiniMax2 (sigmoid, bias for selection, renormalise without bias) and
    SigmoidRenorm (sigmoid, top-k, renormalise), RoutingMethodType comments."""
    rng = np.random.default_rng(300 + E + 50 * use_bias)
    method = orc.MINIMAX2 if use_bias else orc.SIGMOID_RENORM
    for k in range(1, E + 1):
        lg = tie_logits(rng, 3, E)
        bias = (rng.choice(GRID, size=E) / np.float32(2)).astype(np.float32) if use_bias else None
        ids, sc, hard = orc.route(lg, k, method, 1, 1, bias, 1.5)
        assert hard == 0
        for t, (S, kap, w) in enumerate(sigmoid_reference(lg, bias, k, 1.5)):
            assert tuple(sorted(ids[t])) == S, (E, k, t)
            assert ordered_by_key(list(ids[t]), [float(v) for v in kap])
            for j, e in enumerate(ids[t]):
                assert sc[t, j] == pytest.approx(w[e], rel=1e-13)
        assert np.allclose(sc.sum(1), 1.5, rtol=1e-13)


def test_sigmoid_methods_equal_single_group_dsv3(orc):
    """MiniMax2 is DeepSeek-V3's rule with one group (equal up to DeepSeek-V3's
    1e-20 guard), and SigmoidRenorm is MiniMax2 with a zero bias."""
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((64, 32)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, 32).astype(np.float32)
    a = orc.route(lg, 6, orc.MINIMAX2, 1, 1, bias, 2.5)
    b = orc.route(lg, 6, orc.DEEPSEEKV3, 1, 1, bias, 2.5)
    assert np.array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13)
    c = orc.route(lg, 6, orc.SIGMOID_RENORM, 1, 1, None, 2.5)
    d = orc.route(lg, 6, orc.MINIMAX2, 1, 1, np.zeros(32, np.float32), 2.5)
    assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1])


@pytest.mark.parametrize("E", [4, 8, 12])
def test_llama4_brute_force(orc, E):
    """Llama4: top-1 (and, by the same rule, top-k) on the logits, each kept
    expert weighted by its own sigmoid (decimal reference), no renormalisation."""
    rng = np.random.default_rng(400 + E)
    for k in (1, 2, E):
        lg = tie_logits(rng, 4, E)
        ids, sc, _ = orc.route(lg, k, orc.LLAMA4, 1, 1, None, 1.0)
        for t in range(lg.shape[0]):
            keys = [float(v) for v in lg[t]]
            assert tuple(sorted(ids[t])) == brute_topk(keys, k)
            assert ordered_by_key(list(ids[t]), keys)
            for j, e in enumerate(ids[t]):
                assert sc[t, j] == pytest.approx(float(sigmoid_decimal(keys[e])), rel=1e-14)
    lg = np.array([[0.0, 3.0, -1.0, 3.0]], np.float32)
    ids, sc, _ = orc.route(lg, 1, orc.LLAMA4, 1, 1, None, 1.0)
    assert ids.tolist() == [[1]] and sc[0, 0] == pytest.approx(1 / (1 + math.exp(-3.0)), rel=1e-15)


def test_handworked_golden(orc):
    """Hand-derived routing examples (derivations in the fixture file)."""
    path = os.path.join(os.path.dirname(__file__), "golden", "route_handworked.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 4
    for c in cases:
        lg = np.array(c["logits"], np.float32)
        bias = None if c.get("bias") is None else np.array(c["bias"], np.float32)
        ids, sc, _ = orc.route(lg, c["k"], c["method"], c.get("n_group", 1),
                               c.get("topk_group", 1), bias, c.get("scaling", 1.0),
                               c.get("renorm", False))
        assert ids.tolist() == c["ids"], c["name"]
        np.testing.assert_allclose(sc, np.array(c["scales"]), rtol=1e-12, err_msg=c["name"])


def test_rejects_invalid(orc):
    lg = np.zeros((2, 8), np.float32)
    with pytest.raises(ValueError):
        orc.route(lg, 9, orc.DEFAULT)
    with pytest.raises(ValueError):
        orc.route(lg, 2, orc.DEEPSEEKV3, 3, 1)   # 8 % 3 != 0
    with pytest.raises(ValueError):
        orc.route(lg, 5, orc.DEEPSEEKV3, 4, 2)   # k > topk_group * group size
    with pytest.raises(ValueError):
        orc.route(lg, 2, 7)                      # DeepSeekV4: not defined on the pages
