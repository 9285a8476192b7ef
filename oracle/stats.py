"""Host-side load statistics of the routing (oracle; test infrastructure only).

adv12 MoE + EPLB tutorial: §4.2 expert_imbalance, §4.3 eplb_rebalance (LPT
greedy packing), §3.3 the naive contiguous split it is compared against, and
the per-device variance printed in §6.
"""
from __future__ import annotations

import numpy as np


def expert_imbalance(load) -> float:
    """max(load) / (min(load) + 1e-6); the epsilon only guards an empty expert."""
    load = np.asarray(load, dtype=np.float64)
    return float(load.max() / (load.min() + 1e-6))


def lpt_pack(load, D: int):
    """Longest-processing-time-first packing of expert loads onto D devices.

    Experts are taken in order of decreasing load (equal loads: lower expert
    index first); each goes to the currently lightest device (equal device
    loads: lower device index).  Returns (assignment[E] device per expert,
    device_load[D])."""
    load = [int(v) for v in np.asarray(load).ravel()]
    order = sorted(range(len(load)), key=lambda e: (-load[e], e))
    dev = [0] * D
    assignment = [0] * len(load)
    for e in order:
        dmin = min(range(D), key=lambda i: (dev[i], i))
        assignment[e] = dmin
        dev[dmin] += load[e]
    return np.array(assignment, dtype=np.int32), np.array(dev, dtype=np.int64)


def naive_split(load, D: int) -> np.ndarray:
    """Contiguous split: the first E/D experts on device 0, the next on 1, ...
    (tutorial §3.3: experts 0+1 on D0, 2+3 on D1)."""
    load = np.asarray(load, dtype=np.int64)
    E = load.size
    per = -(-E // D)
    return np.array([int(load[i * per:(i + 1) * per].sum()) for i in range(D)], dtype=np.int64)


def sample_variance(v) -> float:
    """Variance with the n-1 denominator: (72, 56) -> 128 and (65, 63) -> 2,
    the two figures the tutorial prints in §6."""
    v = np.asarray(v, dtype=np.float64)
    return float(((v - v.mean()) ** 2).sum() / (v.size - 1))
