"""CPU oracle for the MoE FFN layer forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
__graft_entry__ and the benchmark's CPU-baseline leg may import or call
anything in this package.  The product path (the HIP library and its Python
binding) never does, and shares no code with it.

The oracle is deliberately plain and slow: NumPy in float64, with the layer
computed the way the adv12 MoE + EPLB tutorial draws it (§3.1): a gate Linear,
softmax, top-k, renormalisation, then a loop over experts with a boolean mask
per expert.

Parity status per function (how each is pinned is in tests/test_oracle_pins.py):
  router_logits        pinned (one-hot closed form, shift invariance)
  route                pinned (tutorial Q1 worked example, k=1, k=E, identities)
  select_groups / grouped route   pinned (hand-worked example in tests/golden,
                       all groups = plain routing, one expert per group = plain
                       routing, pairwise group-order brute force)
  bincount             pinned (sum = T*k, tutorial §3.2 total, brute force)
  capacity             pinned (definition bounds, tutorial Q2 example, skew workload value)
  capacity_ranks / dispatch   pinned (tutorial Q2 example, brute-force invariants)
  reroute              pinned (hand-worked examples in tests/golden, zero rounds
                       = drop, unlimited capacity = no-op, capacity / distinctness
                       / exhaustion invariants, a per-expert queue re-statement)
  expert_linear_bias / expert_swiglu   pinned (closed forms)
  forward              pinned (MOE 学习笔记 combine example, dense brute force,
                       identical-expert identity, C=0 / shared-only case,
                       overflow-to-shared closed form)
  stats (imbalance, LPT, naive split, variance)   pinned (tutorial §3.3 / §6 values,
                       4/3 bound against brute-force OPT)
  replicate / eplb_plan   pinned (no replicas = the tutorial's LPT, hand-worked
                       cases in tests/golden, the D'Hondt highest-quotient
                       statement of the replication, placement invariants)
  fp8 e4m3 decode      pinned (OCP format values, torch float8_e4m3fn)
  int8 dequantisation  pinned (code * scale per 128 rows, against torch's int8 cast)
  int4 dequantisation  pinned (hand-worked packed bytes, numpy's arithmetic shifts of
                       the byte for all 256 values, reduction to the int8 case)
  full-size workloads  parity unpinned beyond the invariants above (the pages
                       print no outputs for those shapes)
"""
from .moe_oracle import (  # noqa: F401
    widen, router_logits, select_topk, select_groups, route, route_softmax_of_topk,
    bincount, capacity, capacity_ranks, dispatch, reroute, silu, expert_linear_bias,
    expert_swiglu, forward, forward_tokens, dense_forward, topk_margin,
)
from .stats import (expert_imbalance, lpt_pack, naive_split, sample_variance,  # noqa: F401
                    replicate, replica_loads, eplb_plan)
from .fp8 import e4m3_decode_table, dequant_rows  # noqa: F401
from .int8 import dequant_int8_rows  # noqa: F401
from .int4 import INT4X2, dequant_int4_rows, unpack_int4  # noqa: F401
