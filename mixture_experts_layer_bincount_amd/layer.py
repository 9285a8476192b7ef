"""MoELayer: device buffers plus one moe_forward call per batch.

The layer of the adv12 MoE + EPLB tutorial §4.1 (MoELayer(d_model,
num_experts, top_k) returning the output and the per-expert load), holding
caller-provided device weights.  All compute happens in the HIP library.
"""
from __future__ import annotations

import torch

from . import (DT_BF16, DT_F32, DT_FP8_E4M3, DT_INT4, DT_INT8, LINEAR_BIAS, SWIGLU, make_shape, make_weights,
               moe_forward, moe_pack_router, moe_router_packed_bytes, moe_workspace_bytes)


class MoELayer:
    """Forward pass of one MoE FFN layer on the current HIP device.

    weights: dict of device tensors named as in moe.h (W1, W3, W2 [, s1, s3,
    s2] [, W1s, W3s, W2s [, s1s, s3s, s2s]] for SwiGLU; W, b for Linear+bias).
    overflow: "drop", "reroute" (with reroute_rounds rounds) or "shared", the
    fate of assignments past the capacity.  n_groups / topk_groups: group-
    limited routing (each token uses at most topk_groups groups).  combine:
    "auto", "grouped" or "fused", the form of the combine (moe_combine_form).
    hidden_split: the compensated hidden activation (moe_shape.hidden_split).
    pack_router: split the router's gate once at construction (moe_pack_router)
    instead of in every forward, where the router takes packed weights.
    """

    def __init__(self, T, d, E, top_k, d_ff, *, W_g, b_g=None, weights, capacity=-1,
                 kind="swiglu", w_dtype="bf16", has_shared=False, overflow="drop",
                 reroute_rounds=0, n_groups=0, topk_groups=0, combine="auto", hidden_split=False,
                 pack_router=True, device="cuda"):
        self.kind = SWIGLU if kind == "swiglu" else LINEAR_BIAS
        act = DT_BF16 if self.kind == SWIGLU else DT_F32
        wdt = {"bf16": DT_BF16, "fp8_e4m3": DT_FP8_E4M3, "int8": DT_INT8, "int4": DT_INT4,
               "f32": DT_F32}[w_dtype]
        shape = make_shape(T, d, E, top_k, d_ff, capacity, act, wdt, self.kind, has_shared,
                           overflow, reroute_rounds, n_groups, topk_groups, combine, hidden_split)
        dev = torch.device(device)
        self.W_g = W_g
        self.W_g_packed = None
        if pack_router and moe_router_packed_bytes(shape) > 0:
            # the router's gate split once here, not in every forward
            self.W_g_packed = torch.empty(moe_router_packed_bytes(shape), dtype=torch.uint8,
                                          device=dev)
            moe_pack_router(shape, W_g, self.W_g_packed)
            shape.router_packed = 1
        self.shape = shape
        self.b_g = b_g
        self.weights = make_weights(**weights)
        self.ws = torch.empty(max(moe_workspace_bytes(self.shape), 256), dtype=torch.uint8,
                              device=dev)
        self.y = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
        self.counts = torch.empty((E,), dtype=torch.int32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)

    def forward(self, x: torch.Tensor, stream=None) -> torch.Tensor:
        W_g = self.W_g_packed if self.W_g_packed is not None else self.W_g
        moe_forward(self.shape, x, W_g, self.b_g, self.weights, self.y, self.topk_idx,
                    self.topk_w, self.counts, self.offsets, self.ws, stream)
        return self.y

    __call__ = forward
