"""Pins of the oracle's fp8-activation steps (no GPU).

The quantise-input step of "TensorRT-LLM 源码完全拆解(十三)" (sections
"MoEScheduler:两条执行路径,两套相反的约定" and "“自适应顺序”里的一个细节") and the
fp8 fused MoE of "vLLM 源码完全拆解(八)" (section "量化与 MoE Kernel 选择", after
DeepSeek-V3's fp8 recipe), read as: 1x128 blocks per row, s = fl32(amax/448),
codes = OCP e4m3fn round-to-nearest-even of fl32(v/s), saturating; FC2 reads h
rounded to fp32 and quantised the same way.

Pins: the encoder against torch's float8_e4m3fn cast (a library routine) and a
brute-force nearest-value search; the block quantiser against hand-derived
cases (tests/golden/fp8_quant_handworked.json) and properties that hold for
any input (amax -> 448, half-quantum error bound, power-of-two scale
invariance, block independence); the layer against the bf16-input oracle
when x is already on the fp8 grid, and against a brute-force recomputation
on tiny shapes.
"""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_quant_handworked.json")


def _dec_table(orc):
    return np.array([orc.decode_e4m3(c) for c in range(256)])


def _brute_encode(table, f):
    """Nearest e4m3 value by scanning every code; ties -> even code; the sign
    of zero follows the input; beyond 448 saturates."""
    f = float(np.float32(f))
    best, bd = None, None
    for c in range(256):
        d = table[c]
        if np.isnan(d):
            continue
        if (c & 0x7F) == 0 and c != (0x80 if np.signbit(f) else 0):
            continue
        dist = abs(d - f)
        if bd is None or dist < bd or (dist == bd and (c & 1) == 0):
            best, bd = c, dist
    return best


def _edge_values(table):
    vals = []
    fin = [(c, table[c]) for c in range(256) if not np.isnan(table[c])]
    for c, a in fin:
        vals.append(a)
        if (c & 0x7F) < 0x7E:
            b = table[(c & 0x80) | ((c & 0x7F) + 1)]
            m = np.float32((a + b) / 2)
            vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9 if a >= 0 else -1e9))]
    vals += [448.00003, 449.0, 463.99, 464.0, 470.0, 1e4, -1e4, 1e-30, -1e-30, 0.0, -0.0]
    return np.array(vals, np.float32)


def test_encode_matches_torch_cast(orc):
    """torch's float8_e4m3fn cast rounds to nearest even; clamped to +-448 first
    it is the saturating encoder."""
    table = _dec_table(orc)
    rng = np.random.default_rng(3)
    v = np.concatenate([_edge_values(table),
                        (rng.standard_normal(20000) * np.exp2(rng.integers(-14, 10, 20000))).astype(np.float32)])
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.encode_e4m3(float(f)) for f in v], np.uint8)
    assert np.array_equal(got, ref)


def test_encode_matches_brute_force_nearest(orc):
    table = _dec_table(orc)
    rng = np.random.default_rng(4)
    v = np.concatenate([_edge_values(table),
                        (rng.uniform(-1, 1, 600) * np.exp2(rng.integers(-12, 10, 600))).astype(np.float32)])
    for f in v:
        assert orc.encode_e4m3(float(f)) == _brute_encode(table, f), f


def test_encode_roundtrip_every_code(orc):
    table = _dec_table(orc)
    for c in range(256):
        if np.isnan(table[c]):
            assert orc.encode_e4m3(float("nan")) == 0x7F
            continue
        assert orc.encode_e4m3(float(table[c])) == c


def test_quantize_handworked_golden(orc):
    doc = json.load(open(GOLDEN))
    for case in doc["cases"]:
        x = np.array(case["x"], np.float32)
        q, s = orc.quantize_fp8(x, "f32")
        head = np.array(case["codes_head"], np.uint8)
        n = head.shape[1]
        assert np.array_equal(q[:, :n], head), case["name"]
        assert np.all(q[:, n:] == 0), case["name"]
        assert np.array_equal(s, np.array(case["scales"], np.float32)), case["name"]
        # bf16 input of the same (bf16-exact) values gives the same result
        xb = torch.from_numpy(x).to(torch.bfloat16)
        if torch.equal(xb.float(), torch.from_numpy(x)):
            qb, sb = orc.quantize_fp8(xb.view(torch.int16).numpy(), "bf16")
            assert np.array_equal(qb, q) and np.array_equal(sb, s)


def _bf16_rows(rng, rows, cols):
    mag = np.exp2(rng.integers(-20, 12, (rows, cols // 128, 1)))
    x = (rng.standard_normal((rows, cols // 128, 128)) * mag).reshape(rows, cols)
    return torch.from_numpy(x).to(torch.bfloat16)


def test_quantize_block_properties(orc):
    table = _dec_table(orc)
    rng = np.random.default_rng(5)
    xb = _bf16_rows(rng, 24, 512)
    x = xb.double().numpy()
    q, s = orc.quantize_fp8(xb.view(torch.int16).numpy(), "bf16")
    assert q.shape == (24, 512) and s.shape == (24, 4)
    deq = table[q].reshape(24, 4, 128) * s[:, :, None].astype(np.float64)
    xv = x.reshape(24, 4, 128)
    amax = np.abs(xv).max(axis=2)
    # the largest magnitude of each block lands on +-448
    arg = np.abs(xv).argmax(axis=2)
    for r in range(24):
        for b in range(4):
            assert q[r, b * 128 + arg[r, b]] & 0x7F == 0x7E
    # scale within an fp32 rounding of amax / 448
    assert np.all(np.abs(s.astype(np.float64) - amax / 448) <= amax / 448 * 2.0 ** -23)
    # half-quantum error bound: relative 2^-4 for normal codes, 2^-10 s below
    err = np.abs(deq - xv)
    bound = np.maximum(np.abs(xv) * 2.0 ** -4, s[:, :, None] * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_quantize_power_of_two_invariance_and_block_independence(orc):
    rng = np.random.default_rng(6)
    xb = _bf16_rows(rng, 8, 512)
    q, s = orc.quantize_fp8(xb.view(torch.int16).numpy(), "bf16")
    for j in (-5, 3):
        q2, s2 = orc.quantize_fp8((xb * 2.0 ** j).view(torch.int16).numpy(), "bf16")
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))
    y = xb.clone()
    y[:, 256:384] *= 3
    y[3, 0:128] = 0
    q3, s3 = orc.quantize_fp8(y.view(torch.int16).numpy(), "bf16")
    keep = np.ones(512, bool)
    keep[256:384] = False
    for r in range(8):
        cols = keep.copy()
        if r == 3:
            cols[0:128] = False
        assert np.array_equal(q3[r, cols], q[r, cols])
    assert np.array_equal(np.delete(s3, 2, axis=1)[np.arange(8) != 3], np.delete(s, 2, axis=1)[np.arange(8) != 3])
    assert s3[3, 0] == 0 and np.all(q3[3, :128] == 0)


# ------------------------------------------------------------------- layer
def _weights(rng, G, H, I, wdt):
    w13 = rng.standard_normal((G, 2 * I, H)) / np.sqrt(H)
    w2 = rng.standard_normal((G, H, I)) / np.sqrt(I)
    if wdt == "bf16":
        return (torch.from_numpy(w13).to(torch.bfloat16), torch.from_numpy(w2).to(torch.bfloat16),
                None, None)
    s13 = np.exp2(rng.integers(-9, -5, (G, 2 * I // 128, H // 128))).astype(np.float32)
    s2 = np.exp2(rng.integers(-9, -5, (G, H // 128, I // 128))).astype(np.float32)
    c13 = rng.integers(0, 256, w13.shape).astype(np.uint8)
    c2 = rng.integers(0, 256, w2.shape).astype(np.uint8)
    c13[(c13 & 0x7F) == 0x7F] = 0
    c2[(c2 & 0x7F) == 0x7F] = 0
    return c13, c2, s13, s2


def _deq_w(table, w, s, wdt):
    if wdt == "bf16":
        return w.double().numpy()
    G, R, C = w.shape
    return table[w] * np.repeat(np.repeat(s.astype(np.float64), 128, axis=1), 128, axis=2)[:, :R, :C]


@pytest.mark.parametrize("wdt", ["bf16", "fp8"])
def test_layer_fp8_input_on_grid_matches_unquantised_path(orc, wdt):
    """x already on the fp8 grid (each block holds a +-448 s element, s a
    power of two): quantising x is lossless, so FC1 and h equal the oracle's
    bf16-input ones exactly."""
    rng = np.random.default_rng(7)
    T, H, I, E, k = 5, 256, 256, 3, 2
    codes = rng.integers(0, 256, (T, H)).astype(np.uint8)
    codes[(codes & 0x7F) >= 0x7F] = 0x70
    codes[:, ::128] = 0x7E
    scale = np.exp2(rng.integers(-12, -6, (T, H // 128))).astype(np.float32)
    table = _dec_table(orc)
    x = table[codes] * np.repeat(scale.astype(np.float64), 128, axis=1)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xb.double().numpy(), x)
    q, s = orc.quantize_fp8(xb.view(torch.int16).numpy(), "bf16")
    assert np.array_equal(q, codes) and np.array_equal(s, scale)
    w13, w2, s13, s2 = _weights(rng, E, H, I, wdt)
    W = orc.Weights(w13, w2, wdt, s13, s2)
    ids = np.array([[t % E, (t + 1) % E] for t in range(T)], np.int32)
    off, pp, up = orc.permute(ids, E, 0)
    rows = np.arange(T * k, dtype=np.int32)
    _, h_ref = orc.expert_rows(W, xb.view(torch.int16).numpy(), "bf16", T, k, E, 0, off, pp, rows, want_h=True)
    _, h_a8 = orc.expert_rows(W, q, "fp8", T, k, E, 0, off, pp, rows, want_h=True, x_scale=s)
    assert np.array_equal(h_a8, h_ref)


def _brute_quantize_rows(table, v32):
    rows, cols = v32.shape
    out = np.zeros((rows, cols))
    for r in range(rows):
        for b in range(cols // 128):
            blk = v32[r, b * 128:(b + 1) * 128]
            s = np.float32(np.abs(blk).max()) / np.float32(448)
            for i, f in enumerate(blk):
                c = 0 if s == 0 else _brute_encode(table, np.float32(f) / s)
                out[r, b * 128 + i] = table[c] * float(s)
    return out


@pytest.mark.parametrize("wdt", ["bf16", "fp8"])
def test_layer_fp8_brute_force_tiny(orc, wdt):
    """y_t = sum_j g_j W2 Q(fl32(silu(W1 xq) * W3 xq)) (+ shared) recomputed
    with numpy matmuls and a brute-force nearest-code quantiser."""
    rng = np.random.default_rng(8)
    T, H, I, E, k, n_shared = 3, 128, 256, 2, 2, 1
    table = _dec_table(orc)
    xb = torch.from_numpy(rng.standard_normal((T, H))).to(torch.bfloat16)
    q, s = orc.quantize_fp8(xb.view(torch.int16).numpy(), "bf16")
    w13, w2, s13, s2 = _weights(rng, E + n_shared, H, I, wdt)
    W = orc.Weights(w13, w2, wdt, s13, s2)
    ids = np.array([[0, 1], [1, 0], [1, 0]], np.int32)
    sc = np.array([[0.75, 0.25], [0.6, 0.4], [0.5, 0.5]])
    y = orc.layer_tokens(W, q, "fp8", T, k, E, n_shared, ids, sc, np.arange(T, dtype=np.int32), x_scale=s)
    xq = _brute_quantize_rows(table, xb.float().numpy())
    W13 = _deq_w(table, w13, s13, wdt)
    W2 = _deq_w(table, w2, s2, wdt)
    ref = np.zeros((T, H))
    for t in range(T):
        experts = [(ids[t, j], sc[t, j]) for j in range(k)] + [(E + i, 1.0) for i in range(n_shared)]
        for g, wgt in experts:
            a = W13[g] @ xq[t]
            hpre = a[:I] / (1 + np.exp(-a[:I])) * a[I:]
            hq = _brute_quantize_rows(table, hpre.astype(np.float32)[None, :])[0]
            ref[t] += wgt * (W2[g] @ hq)
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    # the h quantisation is a real step: without it the result moves by ~1e-2
    y_bf = orc.layer_tokens(W, xb.view(torch.int16).numpy(), "bf16", T, k, E, n_shared, ids, sc,
                            np.arange(T, dtype=np.int32))
    assert np.linalg.norm(y_bf - y) / np.linalg.norm(y) > 3e-3
