"""Named workloads and their seeded synthetic inputs.

This module only draws random numbers and rounds them into the storage formats
the layer consumes; it holds none of the layer's arithmetic (no routing, no
permute, no expert FFN, no weighted sum).  Both the HIP path and the CPU oracle
read the tensors it returns, so they always see identical bytes.

Workload shapes follow the models the two teardown pages use as examples:
"TensorRT-LLM 源码完全拆解(十三): MoE 层前向执行" (DeepSeek-V3: 256 routed experts,
top-8, one shared expert, 512 tokens giving 4096 (token, expert) pairs, section
"MoE 在推理侧到底特殊在哪里") and "vLLM 源码完全拆解(八): MoE 层的前向执行"
(Mixtral 8x7B softmax top-k, Qwen3 softmax->top-k->renormalize, section
"FusedTopKRouter").  All values are synthetic; no trained weights are used.

Recipe (per tensor an independent substream, so any expert can be regenerated
alone):
  * x ~ N(0, 1), rounded (RNE) to the activation dtype.
  * W_gate ~ N(0, 1/H) fp32;  logits = fl32(x . W_gate^T), accumulated in fp64
    on the host.  The router projection itself is not part of the path.
  * DeepSeek-V3 shapes: correction bias ~ U(-0.1, 0.1) fp32.
  * Skewed prefill: a seeded random popularity rank r_e in 1..E per expert and
    a logit offset -1.2 ln(r_e) (Zipf-law popularity with exponent 1.2), added
    in fp64 before the single rounding of the logits.
  * w13[g] ~ N(0, 1/H) of shape [2I, H] (gate rows first, then up rows),
    w2[g] ~ N(0, 1/I) of shape [H, I], rounded to the weight dtype.
  * fp8 weights: per 128x128 block of each [out, in] matrix, scale
    s = amax / 448 (fp32, 1.0 for an all-zero block), q = RNE(w / s) clamped to
    +-448, stored as OCP float8 e4m3fn; the dequantised weight is q * s.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Routing method numbering of the RoutingMethodType enum on the TensorRT-LLM
# page (section "路由方法枚举").
ROUTE_DEFAULT = 0
ROUTE_RENORMALIZE = 1
ROUTE_DEEPSEEKV3 = 2
ROUTE_RENORMALIZE_NAIVE = 4
ROUTE_FLAG_RENORMALIZE = 1

# Substream ids.
_TID_X, _TID_WGATE, _TID_BIAS, _TID_ZIPF, _TID_W13, _TID_W2 = range(6)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cid: int                 # substream id of the workload
    T: int
    H: int
    E: int
    I: int
    k: int
    method: int
    flags: int = 0
    n_group: int = 1
    topk_group: int = 1
    scaling: float = 1.0
    n_shared: int = 0
    act: str = "bf16"        # "f32" | "bf16"
    wdt: str = "bf16"        # "f32" | "bf16" | "fp8"
    bias: bool = False
    zipf: float = 0.0        # Zipf exponent of the popularity offsets (0 = none)

    @property
    def G(self) -> int:
        return self.E + self.n_shared

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def R(self) -> int:
        return self.P + self.n_shared * self.T

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 0, T=64, H=256, E=8, I=512, k=2,
                 method=ROUTE_DEFAULT, flags=ROUTE_FLAG_RENORMALIZE,
                 act="f32", wdt="f32"),
        Workload("mixtral_bf16", 1, T=4096, H=4096, E=8, I=14336, k=2,
                 method=ROUTE_RENORMALIZE_NAIVE),
        Workload("dsv3_decode", 2, T=512, H=7168, E=256, I=2048, k=8,
                 method=ROUTE_DEEPSEEKV3, n_group=8, topk_group=4,
                 scaling=2.5, bias=True),
        Workload("dsv3_prefill", 3, T=8192, H=7168, E=256, I=2048, k=8,
                 method=ROUTE_DEEPSEEKV3, n_group=8, topk_group=4,
                 scaling=2.5, bias=True, n_shared=1, zipf=1.2),
        Workload("qwen3_fp8", 4, T=2048, H=4096, E=128, I=1536, k=8,
                 method=ROUTE_RENORMALIZE_NAIVE, wdt="fp8"),
    ]
}

# The DeepSeek-V3 shapes with fp8 e4m3 weights (same seeds and substreams as
# the bf16 ones; weights quantised per 128x128 block): the shapes on which the
# fp8-activation path is measured beside the bf16 headline.
FP8_WORKLOADS = {
    "dsv3_decode_fp8": WORKLOADS["dsv3_decode"].with_(name="dsv3_decode_fp8", wdt="fp8"),
    "dsv3_prefill_fp8": WORKLOADS["dsv3_prefill"].with_(name="dsv3_prefill_fp8", wdt="fp8"),
}


def get(name: str) -> Workload:
    """A workload of WORKLOADS or FP8_WORKLOADS by name."""
    return WORKLOADS[name] if name in WORKLOADS else FP8_WORKLOADS[name]


TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16,
               "fp8": torch.float8_e4m3fn}
FP8_MAX = 448.0
QBLOCK = 128


def _rng(seed: int, cid: int, tid: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, tid, expert])))


def _torch_gen(seed: int, cid: int, tid: int, expert: int, device) -> torch.Generator:
    s = int(np.random.SeedSequence([seed, cid, tid, expert]).generate_state(1, np.uint64)[0])
    g = torch.Generator(device=device)
    g.manual_seed(s & ((1 << 63) - 1))
    return g


def make_x(w: Workload, seed: int = 0) -> torch.Tensor:
    """Token activations [T, H] on the host, rounded to the activation dtype."""
    x = _rng(seed, w.cid, _TID_X).standard_normal((w.T, w.H), dtype=np.float32)
    return torch.from_numpy(x).to(TORCH_DTYPE[w.act])


def make_x_device(w: Workload, seed: int = 0, device="cuda", chunk_rows: int = 8192) -> torch.Tensor:
    """Token activations [T, H] drawn N(0, 1) directly on `device` (seeded torch
    generator, in row chunks) and rounded to the activation dtype: for shapes
    whose host draw would be too large.  Other values than make_x's."""
    x = torch.empty((w.T, w.H), dtype=TORCH_DTYPE[w.act], device=device)
    gen = _torch_gen(seed, w.cid, _TID_X, 0, device)
    for r0 in range(0, w.T, chunk_rows):
        r1 = min(w.T, r0 + chunk_rows)
        x[r0:r1] = torch.randn((r1 - r0, w.H), generator=gen, device=device, dtype=torch.float32)
    return x


def make_logits_direct(w: Workload, seed: int = 0) -> torch.Tensor:
    """Router logits [T, E] drawn N(0, 1) directly (fp32, host), for shapes
    where forming x . W_gate^T on the host would be too large."""
    lg = _rng(seed, w.cid, _TID_WGATE).standard_normal((w.T, w.E), dtype=np.float32)
    return torch.from_numpy(lg)


def make_bias(w: Workload, seed: int = 0) -> Optional[torch.Tensor]:
    if not w.bias:
        return None
    b = _rng(seed, w.cid, _TID_BIAS).uniform(-0.1, 0.1, size=w.E).astype(np.float32)
    return torch.from_numpy(b)


def zipf_offsets(w: Workload, seed: int = 0) -> Optional[np.ndarray]:
    if not w.zipf:
        return None
    rank = _rng(seed, w.cid, _TID_ZIPF).permutation(w.E) + 1
    return -w.zipf * np.log(rank.astype(np.float64))


def make_logits(w: Workload, x: torch.Tensor, seed: int = 0) -> torch.Tensor:
    """Router logits fl32(x . W_gate^T (+ popularity offset)), fp64 accumulate."""
    wg = _rng(seed, w.cid, _TID_WGATE).standard_normal((w.E, w.H), dtype=np.float32)
    wg = (wg * np.float32(math.sqrt(1.0 / w.H))).astype(np.float32)
    xd = x.to(torch.float64).numpy()
    acc = xd @ wg.astype(np.float64).T
    off = zipf_offsets(w, seed)
    if off is not None:
        acc = acc + off[None, :]
    return torch.from_numpy(acc.astype(np.float32))


def quantize_fp8_blockwise(wf: torch.Tensor):
    """[rows, cols] fp32 -> (q float8_e4m3fn [rows, cols], s fp32 [rows/128, cols/128])."""
    rows, cols = wf.shape
    blk = wf.reshape(rows // QBLOCK, QBLOCK, cols // QBLOCK, QBLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    qf = (blk / s[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    q = qf.reshape(rows, cols).to(torch.float8_e4m3fn)
    return q, s


def _expert_matrix(w: Workload, seed: int, tid: int, g: int, shape, std: float, device):
    gen = _torch_gen(seed, w.cid, tid, g, device)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def make_weights(w: Workload, seed: int = 0, device="cpu"):
    """(w13 [G, 2I, H], w2 [G, H, I], w13_scale, w2_scale) on `device`.

    Scales are None unless the weight dtype is fp8.  Group g < E is routed
    expert g; group E + s is shared expert s.  Each group is drawn from its own
    substream, directly on `device`, so the largest shapes never need a host
    copy of all weights.
    """
    G, H, I = w.G, w.H, w.I
    dt = TORCH_DTYPE[w.wdt]
    w13 = torch.empty((G, 2 * I, H), dtype=dt, device=device)
    w2 = torch.empty((G, H, I), dtype=dt, device=device)
    s13 = s2 = None
    if w.wdt == "fp8":
        s13 = torch.empty((G, 2 * I // QBLOCK, H // QBLOCK), dtype=torch.float32, device=device)
        s2 = torch.empty((G, H // QBLOCK, I // QBLOCK), dtype=torch.float32, device=device)
    for g in range(G):
        a = _expert_matrix(w, seed, _TID_W13, g, (2 * I, H), math.sqrt(1.0 / H), device)
        b = _expert_matrix(w, seed, _TID_W2, g, (H, I), math.sqrt(1.0 / I), device)
        if w.wdt == "fp8":
            w13[g], s13[g] = quantize_fp8_blockwise(a)
            w2[g], s2[g] = quantize_fp8_blockwise(b)
        else:
            w13[g] = a.to(dt)
            w2[g] = b.to(dt)
    return w13, w2, s13, s2


def make_inputs(w: Workload, seed: int = 0, device="cpu"):
    """All inputs of one workload: dict of x, logits, bias, w13, w2, w13_scale, w2_scale.

    x, logits and bias are built on the host (fp64 router projection) and then
    moved to `device`; weights are drawn on `device`.
    """
    x = make_x(w, seed)
    logits = make_logits(w, x, seed)
    bias = make_bias(w, seed)
    w13, w2, s13, s2 = make_weights(w, seed, device)
    mv = (lambda t: None if t is None else t.to(device))
    return dict(x=mv(x), logits=mv(logits), bias=mv(bias), w13=w13, w2=w2,
                w13_scale=s13, w2_scale=s2)
