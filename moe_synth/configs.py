"""Workload presets for the MoE layer forward pass.

Five workloads: the tutorial-sized fp32 layer (the adv12 MoE + EPLB tutorial,
§3.1: 64 tokens, width 8, 4 experts, top-2, Linear experts with bias), a
Mixtral-shaped prefill layer, the same layer at decode size, a fine-grained
layer with a shared expert (DeepSeek-style: 256 routed experts + 1 shared,
top-8, as listed in the tutorial's §5 table and on the iopenshare page §1.4),
and a capacity-limited, skewed layer.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

SEED_BASE = 20261203


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens on this GPU
    d: int            # model width
    E: int            # routed experts
    k: int            # experts kept per token
    d_ff: int         # expert hidden width (0 for the Linear+bias expert)
    kind: str         # "linear_bias" | "swiglu"
    act: str          # activation / x dtype: "f32" | "bf16"
    w: str            # expert weight dtype: "f32" | "bf16" | "fp8_e4m3" | "int8" | "int4"
    cf: Optional[float] = None       # capacity factor; None = unlimited
    router_bias: Optional[str] = None  # None | "zipf1.5": b_e = 1.5*ln(1/(e+1))
    shared: bool = False             # one always-on shared expert
    seed: int = SEED_BASE
    x_from: Optional[str] = None     # take x as the first T rows of this config's x
    w_from: Optional[str] = None     # take all weights from this config
    hidden_split: bool = False       # the layer keeps its hidden activation as two bf16 terms

    @property
    def A(self) -> int:
        """Number of (token, slot) assignments."""
        return self.T * self.k

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": MoEConfig("tiny", T=64, d=8, E=4, k=2, d_ff=0, kind="linear_bias",
                      act="f32", w="f32", seed=SEED_BASE + 1),
    "mixtral": MoEConfig("mixtral", T=4096, d=4096, E=8, k=2, d_ff=14336,
                         kind="swiglu", act="bf16", w="bf16", seed=SEED_BASE + 2),
    "decode": MoEConfig("decode", T=64, d=4096, E=8, k=2, d_ff=14336,
                        kind="swiglu", act="bf16", w="bf16", seed=SEED_BASE + 2,
                        x_from="mixtral", w_from="mixtral"),
    "decode_fp8": MoEConfig("decode_fp8", T=64, d=4096, E=8, k=2, d_ff=14336,
                            kind="swiglu", act="bf16", w="fp8_e4m3", seed=SEED_BASE + 2,
                            x_from="mixtral", w_from="mixtral"),
    "decode_int8": MoEConfig("decode_int8", T=64, d=4096, E=8, k=2, d_ff=14336,
                             kind="swiglu", act="bf16", w="int8", seed=SEED_BASE + 2,
                             x_from="mixtral", w_from="mixtral"),
    "decode_int4": MoEConfig("decode_int4", T=64, d=4096, E=8, k=2, d_ff=14336,
                             kind="swiglu", act="bf16", w="int4", seed=SEED_BASE + 2,
                             x_from="mixtral", w_from="mixtral"),
    "fine_grained": MoEConfig("fine_grained", T=4096, d=7168, E=256, k=8,
                              d_ff=2048, kind="swiglu", act="bf16", w="bf16",
                              shared=True, seed=SEED_BASE + 4),
    "fine_grained_fp8": MoEConfig("fine_grained_fp8", T=4096, d=7168, E=256,
                                  k=8, d_ff=2048, kind="swiglu", act="bf16",
                                  w="fp8_e4m3", shared=True, seed=SEED_BASE + 4),
    "fine_grained_int8": MoEConfig("fine_grained_int8", T=4096, d=7168, E=256,
                                   k=8, d_ff=2048, kind="swiglu", act="bf16",
                                   w="int8", shared=True, seed=SEED_BASE + 4),
    "fine_grained_int4": MoEConfig("fine_grained_int4", T=4096, d=7168, E=256,
                                   k=8, d_ff=2048, kind="swiglu", act="bf16",
                                   w="int4", shared=True, seed=SEED_BASE + 4),
    "capacity_skew": MoEConfig("capacity_skew", T=16384, d=4096, E=64, k=2,
                               d_ff=1408, kind="swiglu", act="bf16", w="bf16",
                               cf=1.25, router_bias="zipf1.5",
                               seed=SEED_BASE + 5, hidden_split=True),
}


def get_config(name: str) -> MoEConfig:
    return CONFIGS[name]


def custom_config(T, d, E, k, d_ff=0, *, kind="swiglu", act="bf16", w="bf16",
                  cf=None, router_bias=None, shared=False, seed=12345,
                  name="custom", hidden_split=False) -> MoEConfig:
    return MoEConfig(name, T=T, d=d, E=E, k=k, d_ff=d_ff, kind=kind, act=act,
                     w=w, cf=cf, router_bias=router_bias, shared=shared,
                     seed=seed, hidden_split=hidden_split)
