"""The four-call MoE layer forward with buffers allocated once.

route -> permute -> expert_ffn (FC1 + SwiGLU, FC2) -> finalize, all enqueued on
torch's current stream; nothing is read back to the host between calls.  With
fp8_act=True (bf16 x, fp8 weights) the FFN step is quantize_fp8(x) followed by
expert_ffn_fp8.  With fused=True the FFN step is the one-kernel form with h kept
on chip (expert_ffn_fused / expert_ffn_fp8_fused: same results, no workspace
for h).
"""
from __future__ import annotations

import torch

from . import binding as B


class MoELayer:
    """Shapes and routing settings of one layer plus its preallocated buffers."""

    def __init__(self, T, H, I, E, k, method, act_dtype=torch.bfloat16, n_group=1,
                 topk_group=1, scaling=1.0, renormalize=False, n_shared=0, device="cuda",
                 fp8_act=False, fused=False, split=0):
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.method, self.n_group, self.topk_group = method, n_group, topk_group
        self.scaling, self.renormalize, self.n_shared = scaling, renormalize, n_shared
        self.act = act_dtype
        self.fp8_act = fp8_act
        self.fused, self.split = fused, split
        if fp8_act and act_dtype != torch.bfloat16:
            raise ValueError("fp8 activations take a bf16 layer input")
        if fused and act_dtype != torch.bfloat16:
            raise ValueError("the fused FFN takes a bf16 layer input")
        G, P = E + n_shared, T * k
        R = P + n_shared * T
        d = torch.device(device)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=d)
        self.scales = torch.empty((T, k), dtype=torch.float32, device=d)
        self.offsets = torch.empty(G + 1, dtype=torch.int32, device=d)
        self.permuted_pair = torch.empty(P, dtype=torch.int32, device=d)
        self.unpermute = torch.empty(P, dtype=torch.int32, device=d)
        self.fc2_out = torch.empty((R, H), dtype=act_dtype, device=d)
        self.y = torch.empty((T, H), dtype=act_dtype, device=d)
        # fused: the workspace only serves the permute (h stays on chip)
        self.ws = B.alloc_workspace(T, k, E, n_shared, 128 if fused else H, 128 if fused else I,
                                    torch.float8_e4m3fn if fp8_act else act_dtype, d)
        if fp8_act:
            self.xq = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=d)
            self.x_scale = torch.empty((T, H // 128), dtype=torch.float32, device=d)

    def forward(self, x, logits, w13, w2, bias=None, w13_scale=None, w2_scale=None):
        """y [T, H] for x [T, H] and router logits [T, E] (fp32).  The result is
        the layer's own output buffer: the next call overwrites it, so clone it
        to keep it."""
        B.route(logits, self.k, self.method, self.n_group, self.topk_group, bias, self.scaling,
                self.renormalize, out=(self.ids, self.scales))
        B.permute(self.ids, self.E, self.n_shared, ws=self.ws,
                  out=(self.offsets, self.permuted_pair, self.unpermute))
        if self.fp8_act:
            B.quantize_fp8(x, out=(self.xq, self.x_scale))
            if self.fused:
                B.expert_ffn_fp8_fused(self.xq, self.x_scale, self.offsets, self.permuted_pair,
                                       w13, w2, w13_scale, w2_scale, self.k, self.E,
                                       self.n_shared, split=self.split, out=self.fc2_out)
            else:
                B.expert_ffn_fp8(self.xq, self.x_scale, self.offsets, self.permuted_pair, w13,
                                 w2, w13_scale, w2_scale, self.k, self.E, self.n_shared,
                                 ws=self.ws, out=self.fc2_out)
        elif self.fused:
            B.expert_ffn_fused(x, self.offsets, self.permuted_pair, w13, w2, self.k, self.E,
                               self.n_shared, w13_scale, w2_scale, split=self.split,
                               out=self.fc2_out)
        else:
            B.expert_ffn(x, self.offsets, self.permuted_pair, w13, w2, self.k, self.E,
                         self.n_shared, w13_scale, w2_scale, ws=self.ws, out=self.fc2_out)
        B.finalize(self.fc2_out, self.unpermute, self.scales, self.n_shared, out=self.y)
        return self.y

    __call__ = forward


def layer_for_workload(w, device="cuda", fp8_act=False, fused=False, split=0) -> MoELayer:
    """MoELayer configured for a workloads.Workload."""
    return MoELayer(w.T, w.H, w.I, w.E, w.k, w.method,
                    torch.float32 if w.act == "f32" else torch.bfloat16, w.n_group,
                    w.topk_group, w.scaling, bool(w.flags & B.ROUTE_FLAG_RENORMALIZE),
                    w.n_shared, device, fp8_act, fused, split)
