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


def replicate(load, D: int, extra: int):
    """Hot-expert replication: replicas per expert.

    fde-learning "MoE 并行" (通信瓶颈的缓解策略, Expert 复制: a popular
    expert gets a copy on several GPUs) and the tutorial's online EPLB (§5:
    monitor, then move hot experts).  Read as: every expert starts with one
    replica; `extra` times, the expert with the largest load per replica
    (load / replicas, compared exactly; equal: the lower expert) gets one
    more, among the experts that have fewer than D replicas (one per device
    at most).  Returns replicas[E]."""
    from fractions import Fraction
    load = [int(v) for v in np.asarray(load).ravel()]
    r = [1] * len(load)
    for _ in range(extra):
        cands = [e for e in range(len(load)) if r[e] < D]
        if not cands:
            break
        best = max(cands, key=lambda e: (Fraction(load[e], r[e]), -e))
        r[best] += 1
    return np.array(r, dtype=np.int64)


def replica_loads(load_e: int, r: int):
    """An expert's tokens split as evenly as possible over its r replicas:
    the first load % r replicas take one token more."""
    return [load_e // r + (1 if i < load_e % r else 0) for i in range(r)]


def eplb_plan(load, D: int, extra: int):
    """Placement of the replicas on D devices: LPT over the replicas.

    The replicas (replicate(), loads by replica_loads()) are taken in order
    of decreasing load (equal: lower expert, then lower replica); each goes
    to the lightest device that does not hold a replica of the same expert
    yet (equal loads: lower device) -- the tutorial's LPT (§3.3, §4.3) with
    the copies of one expert on different devices.  Slots are numbered
    expert by expert, replica by replica.  Returns dict(replicas[E],
    slot_expert[S], slot_load[S], slot_device[S], device_load[D])."""
    load = [int(v) for v in np.asarray(load).ravel()]
    r = replicate(load, D, extra)
    slots = [(e, i, l) for e in range(len(load)) for i, l in enumerate(replica_loads(load[e], int(r[e])))]
    order = sorted(range(len(slots)), key=lambda s: (-slots[s][2], slots[s][0], slots[s][1]))
    dev = [0] * D
    holds = [set() for _ in range(D)]
    slot_device = [-1] * len(slots)
    for s in order:
        e, _, l = slots[s]
        d = min((i for i in range(D) if e not in holds[i]), key=lambda i: (dev[i], i))
        slot_device[s] = d
        holds[d].add(e)
        dev[d] += l
    return dict(replicas=r,
                slot_expert=np.array([s[0] for s in slots], dtype=np.int64),
                slot_load=np.array([s[2] for s in slots], dtype=np.int64),
                slot_device=np.array(slot_device, dtype=np.int64),
                device_load=np.array(dev, dtype=np.int64))
