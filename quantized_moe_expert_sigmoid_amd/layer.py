"""One routed-expert MoE layer held in HBM, run through the C ABI.

The hot path of a call (all on the context stream, no host round trip):
    moe_quantize_act_i8 -> moe_router_topk -> moe_expert_ffn_q{4,8,2}
    -> moe_combine
Weights enter as fp32 host arrays and are quantised and packed on the GPU
(moe_quantize_rows) straight into contiguous per-expert blocks.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (FFN_BY_BITS, ExpertBlocks, MoeCtx, moe_combine, moe_layer_forward, moe_quantize_act_i8,
               moe_router_topk)


def _to_dev(a, device):
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=torch.float32).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class MoeLayer:
    def __init__(self, ctx: MoeCtx, H: int, I: int, E: int, k: int, bits: int = 4, has_shared: bool = True,
                 routed_scale: float = 1.0, device: str = "cuda", top_p: float = 0.0):
        self.ctx, self.H, self.I, self.E, self.k, self.bits = ctx, H, I, E, k, bits
        self.routed_scale = routed_scale
        self.top_p = top_p  # 0: keep all k experts (see moe_router_cfg)
        self.device = device
        self.experts = ExpertBlocks(E, bits, H, I, device)
        self.shared = ExpertBlocks(1, bits, H, I, device) if has_shared else None
        self.w_router = torch.zeros((E, H), dtype=torch.float32, device=device)
        self.bias = None
        self._bufs = {}

    # -- weights -----------------------------------------------------------
    def set_expert_fp32(self, e: int, wg, wu, wd):
        self.experts.pack_from_fp32(self.ctx, e, _to_dev(wg, self.device), _to_dev(wu, self.device),
                                    _to_dev(wd, self.device))

    def set_shared_fp32(self, wg, wu, wd):
        self.shared.pack_from_fp32(self.ctx, 0, _to_dev(wg, self.device), _to_dev(wu, self.device),
                                   _to_dev(wd, self.device))

    def set_router(self, w_router, bias=None):
        self.w_router = _to_dev(w_router, self.device)
        self.bias = None if bias is None else _to_dev(bias, self.device)

    # -- buffers -----------------------------------------------------------
    def buffers(self, T: int):
        b = self._bufs.get(T)
        if b is None:
            d, H, k = self.device, self.H, self.k
            b = dict(xq=torch.empty((T, H), dtype=torch.int8, device=d),
                     sx=torch.empty((T,), dtype=torch.float32, device=d),
                     idx=torch.empty((T, k), dtype=torch.int32, device=d),
                     w=torch.empty((T, k), dtype=torch.float32, device=d),
                     y=torch.zeros((T, k + 1, H), dtype=torch.float32, device=d),
                     out=torch.empty((T, H), dtype=torch.float32, device=d))
            self._bufs[T] = b
        return b

    # -- forward -----------------------------------------------------------
    def forward(self, x: torch.Tensor, logits: torch.Tensor | None = None) -> dict:
        """The whole layer in one library call (moe_layer_forward). x: fp32
        [T][H] device tensor; logits (optional) fp32 [T][E] to route on given
        logits instead of the router weights. Returns the buffers (out, idx,
        w, xq, sx, y)."""
        T = x.shape[0]
        b = self.buffers(T)
        sh = self.shared.struct(0) if self.shared is not None else None
        moe_layer_forward(self.ctx, self.bits, x, self.experts.table, sh, self.k, self.I, b["out"],
                          w_router=None if logits is not None else self.w_router, bias=self.bias, logits=logits,
                          routed_scale=self.routed_scale, top_p=self.top_p, topk_idx=b["idx"], topk_w=b["w"],
                          xq=b["xq"], sx=b["sx"],
                          y_slots=b["y"])
        return b

    def forward_steps(self, x: torch.Tensor, logits: torch.Tensor | None = None) -> dict:
        """The same layer through the per-step entry points: moe_quantize_act_i8
        -> moe_router_topk -> moe_expert_ffn_q* -> moe_combine."""
        T = x.shape[0]
        b = self.buffers(T)
        ctx = self.ctx
        moe_quantize_act_i8(ctx, x, b["xq"], b["sx"])
        if logits is not None:
            moe_router_topk(ctx, logits, None, self.bias, self.k, b["idx"], b["w"], self.routed_scale,
                            logits_in=True, top_p=self.top_p)
        else:
            moe_router_topk(ctx, x, self.w_router, self.bias, self.k, b["idx"], b["w"], self.routed_scale,
                            top_p=self.top_p)
        sh = self.shared.struct(0) if self.shared is not None else None
        FFN_BY_BITS[self.bits](ctx, self.experts.table, sh, None, b["xq"], b["sx"], b["idx"], self.H, self.I, self.E,
                               b["y"])
        moe_combine(ctx, b["y"], b["w"], self.shared is not None, b["out"])
        return b
