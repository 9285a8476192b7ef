"""Plain CPU oracle of the MoE FFN layer forward pass (test infrastructure only).

Every step is written the plainest way, in float64, in the order the pages
give it:

  router      logits = x . W_g (+ b)            iopenshare "MoE 混合专家架构" §2.1
                                                (TopKGating: gate Linear, no bias);
                                                adv12 tutorial §3.1 / §4.1
  top-k       keep the k experts with the largest logits (ties: lower index);
              optionally only among the experts of the token's best groups
              (group-limited routing)          fde-learning "MoE 并行"
                                                (Hierarchical Routing); tutorial
                                                §5 (device-limited routing)
  weights     softmax over all experts, keep the k selected probabilities and
              divide by their sum                tutorial §4.1 table steps 1-3, Q1
  bincount    load[e] = number of (token, slot) pairs routed to e    tutorial §3.2
  capacity    C = ceil(cf * T * k / E); assignments past C in token order are
              dropped and add nothing (their token keeps the residual path)
                                                fde-learning "MoE 并行", Capacity
                                                Factor; tutorial Q2
  overflow    instead of dropping (a policy, "drop" by default):
              "reroute": in rounds, every dropped assignment moves to its
              token's next-ranked unused expert; an expert accepts the round's
              requests in token order while it has capacity left
                                                fde-learning "MoE 并行", 推理时
                                                的负载均衡 (dynamic re-routing)
              "shared": a dropped assignment's weight goes to the shared
              expert                            tutorial Q2 (overflow to the
                                                shared expert)
  experts     for e in experts: mask = (topk_idx == e) & kept;
              out[mask] += w * expert_e(x[mask])  tutorial §3.1 diagram
  shared      y += shared_expert(x) for every token, weight 1
                                                iopenshare §1.4 (always-active
                                                shared experts)

Inputs: x as float32 or bfloat16 bit patterns (uint16); W_g float32 [d, E];
expert weights output-major ([out, in]) as float32, bf16 bits, fp8 e4m3
codes (uint8), symmetric int8 codes (int8) or packed symmetric int4 codes
(the INT4X2 dtype, [out, in/2]), the codes with float32 scales per 128 output
features.
"""
from __future__ import annotations

import math

import numpy as np

from .fp8 import dequant_rows
from .int4 import dequant_int4_rows, is_int4x2
from .int8 import dequant_int8_rows


# ---------------------------------------------------------------- numerics
def widen(a: np.ndarray) -> np.ndarray:
    """Exact conversion to float64.  uint16 arrays are bfloat16 bit patterns
    (the upper half of an IEEE binary32)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _weight(w: dict, name: str) -> np.ndarray:
    """One expert matrix in float64; fp8 (uint8), int8 or packed int4 codes are
    decoded and scaled exactly."""
    a = w[name]
    if is_int4x2(a):
        return dequant_int4_rows(a, w["s" + name[1:]])
    if a.dtype == np.uint8:
        return dequant_rows(a, w["s" + name[1:]])
    if a.dtype == np.int8:
        return dequant_int8_rows(a, w["s" + name[1:]])
    return widen(a)


# ---------------------------------------------------------------- router
def router_logits(x: np.ndarray, W_g: np.ndarray, b_g=None) -> np.ndarray:
    """Gate Linear without bias (iopenshare §2.1 TopKGating; tutorial §4.1),
    plus an optional per-expert bias.  Computed in float64, returned as the
    float32 logits the routing step consumes."""
    logits = widen(x) @ np.asarray(W_g, dtype=np.float64)
    if b_g is not None:
        logits = logits + np.asarray(b_g, dtype=np.float64)[None, :]
    return logits.astype(np.float32)


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, slot 0 the largest.

    Ties go to the lower expert index.  -0.0 and +0.0 compare equal (IEEE
    comparison), so they tie as well.  Selection is done on the logits:
    softmax is monotone, so this is the same set as selecting on the softmax
    scores (tutorial §3.1) and as torch.topk on logits (iopenshare §2.1)."""
    logits = np.asarray(logits, dtype=np.float64) + 0.0  # -0.0 -> +0.0
    T, E = logits.shape
    e_idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((e_idx, -logits), axis=-1)  # primary: -logit, then index
    return order[:, :k].astype(np.int32)


def weights_for(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Routing weights of the selected experts: softmax over all E experts
    (maximum subtracted first, the safe softmax of iopenshare §4.2), then the
    selected probabilities divided by their sum (tutorial Q1)."""
    l64 = np.asarray(logits, dtype=np.float64)
    z = l64 - l64.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def select_groups(logits: np.ndarray, groups: int, topk_groups: int) -> np.ndarray:
    """Group-limited routing, step 1: which expert groups each token may use.

    fde-learning "MoE 并行" (通信瓶颈的缓解策略, Hierarchical Routing: choose
    a group first, then an expert) and the tutorial's DeepSeek-V3 notes
    (device-limited routing: a token's experts lie on at most M devices).
    The E experts form `groups` equal groups of consecutive indices; a
    group's score for a token is its largest logit; the token keeps the
    `topk_groups` groups with the largest scores (equal scores: the lower
    group first).  Returns a bool mask [T, groups]."""
    l64 = np.asarray(logits, dtype=np.float64) + 0.0
    T, E = l64.shape
    score = l64.reshape(T, groups, E // groups).max(axis=2)
    g_idx = np.broadcast_to(np.arange(groups), (T, groups))
    order = np.lexsort((g_idx, -score), axis=-1)[:, :topk_groups]
    mask = np.zeros((T, groups), dtype=bool)
    np.put_along_axis(mask, order, True, axis=1)
    return mask


def route(logits: np.ndarray, k: int, groups: int = 0, topk_groups: int = 0):
    """(topk_idx [T,k] int32, topk_w [T,k] float64).  With groups > 1 the
    top-k is taken among the experts of the kept groups only
    (select_groups); the weights follow the same rule as without groups."""
    if groups > 1:
        T, E = logits.shape
        allowed = np.repeat(select_groups(logits, groups, topk_groups), E // groups, axis=1)
        masked = np.where(allowed, np.asarray(logits, dtype=np.float64), -np.inf)
        idx = select_topk(masked, k)
    else:
        idx = select_topk(logits, k)
    return idx, weights_for(logits, idx)


def route_softmax_of_topk(logits: np.ndarray, k: int):
    """The other formulation on the pages: softmax of the k selected logits
    (iopenshare §2.1 TopKGating and §4.2 safe_topk_routing).  Mathematically
    equal to route(); kept as an independent cross-check."""
    idx = select_topk(logits, k)
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return idx, z / z.sum(axis=1, keepdims=True)


def topk_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """min over j=1..k of (l_(j) - l_(j+1)) on the sorted float32 logits of each
    token; the j=k gap is skipped when k equals E.  Tokens with a small margin
    may legitimately change their selection under a different fp32
    summation order of the router."""
    s = -np.sort(-np.asarray(logits, dtype=np.float64), axis=1)
    E = s.shape[1]
    last = min(k, E - 1)
    if last == 0:
        return np.full(s.shape[0], np.inf)
    gaps = s[:, :last] - s[:, 1:last + 1]
    return gaps.min(axis=1)


# ---------------------------------------------------------------- load accounting
def bincount(idx: np.ndarray, E: int) -> np.ndarray:
    """load[e]: how many (token, slot) pairs chose expert e (tutorial §3.2)."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int64)


def capacity(T: int, E: int, k: int, cf) -> int:
    """Tokens an expert may take: ceil(cf * T * k / E), evaluated in IEEE
    double in this order; -1 (unlimited) when cf is None or <= 0.

    The capacity factor is max_tokens_per_expert / (tokens / experts) on the
    fde-learning page (Capacity Factor); with top-k routing the tokens an
    expert sees are the T*k assignments, hence the k."""
    if cf is None or cf <= 0:
        return -1
    return int(math.ceil((float(cf) * float(T * k)) / float(E)))


def capacity_ranks(idx: np.ndarray, E: int) -> np.ndarray:
    """rank[t, j]: how many earlier tokens t' < t also chose expert idx[t, j].
    A plain walk in token order; a token never picks one expert twice.
    Entries -1 (no expert) get rank -1 and are not counted."""
    T, k = idx.shape
    seen = np.zeros(E, dtype=np.int64)
    rank = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                rank[t, j] = -1
                continue
            rank[t, j] = seen[e]
            seen[e] += 1
    return rank


def dispatch(idx: np.ndarray, w: np.ndarray, E: int, C: int):
    """Group the kept assignments by expert, in token order within an expert.

    Returns a dict with counts[E], kept[E], offsets[E+1] (exclusive prefix sum
    of kept), keep[T,k] bool, rank[T,k], perm_token[P], perm_slot[P],
    perm_w[P] and slot_pos[T,k] (position in the grouped order, -1 if
    dropped).  Dropped assignments add nothing (tutorial Q2: overflow is
    dropped; fde-learning: overflow takes the residual path).  idx entries -1
    stand for assignments already dropped (no expert)."""
    T, k = idx.shape
    counts = bincount(idx[idx >= 0], E)
    rank = capacity_ranks(idx, E)
    if C < 0:
        keep = idx >= 0
        kept = counts.copy()
    else:
        keep = (idx >= 0) & (rank < C)
        kept = np.minimum(counts, C)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    P = int(offsets[-1])
    perm_token = np.full(P, -1, dtype=np.int64)
    perm_slot = np.full(P, -1, dtype=np.int64)
    perm_w = np.zeros(P, dtype=np.float64)
    slot_pos = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                e = int(idx[t, j])
                pos = int(offsets[e] + rank[t, j])
                perm_token[pos] = t
                perm_slot[pos] = j
                perm_w[pos] = w[t, j]
                slot_pos[t, j] = pos
    return dict(counts=counts, kept=kept, offsets=offsets, keep=keep, rank=rank,
                perm_token=perm_token, perm_slot=perm_slot, perm_w=perm_w,
                slot_pos=slot_pos, C=C)


def reroute(logits: np.ndarray, idx: np.ndarray, E: int, C: int, rounds: int) -> np.ndarray:
    """Overflow re-routing: the final expert of every (token, slot), -1 for an
    assignment that stays dropped.

    fde-learning "MoE 并行" (推理时的负载均衡): when an expert is over its
    capacity, the token is routed to the next expert.  Read here as rounds:
    the first pass keeps, per expert, the first C assignments in token order
    (as dispatch()); then in each round every still-dropped assignment, taken
    in token order and slot order, requests its token's next ranked expert
    that the token has not used or requested yet (ranks by logit, ties to the
    lower index, as select_topk), and each expert accepts requests in that
    order while it has capacity left.  Requests that find the expert full
    wait for the next round.  After `rounds` rounds the rest are dropped."""
    T, k = idx.shape
    if C < 0:
        return np.asarray(idx, dtype=np.int64).copy()
    ranked = select_topk(logits, E)
    rank = capacity_ranks(idx, E)
    final = np.where(rank < C, idx, -2).astype(np.int64)  # -2: waiting
    used = np.minimum(bincount(idx, E), C)
    nxt = np.full(T, k, dtype=np.int64)  # next unused position in ranked[t]
    for _ in range(rounds):
        requests = []
        for t in range(T):
            for j in range(k):
                if final[t, j] == -2 and nxt[t] < E:
                    requests.append((t, j, int(ranked[t, nxt[t]])))
                    nxt[t] += 1
        for t, j, e in requests:
            if used[e] < C:
                final[t, j] = e
                used[e] += 1
    final[final == -2] = -1
    return final


# ---------------------------------------------------------------- experts
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def expert_linear_bias(X: np.ndarray, w: dict) -> np.ndarray:
    """The tutorial's expert, nn.Linear(d, d) with bias (tutorial §4.1):
    X . W^T + b with W stored [out, in]."""
    return X @ _weight(w, "W").T + widen(w["b"])[None, :]


def expert_swiglu(X: np.ndarray, w: dict) -> np.ndarray:
    """SiLU-gated FFN: silu(X . W1^T) * (X . W3^T), then . W2^T.
    iopenshare §5.2 applies silu to the W1 product; W3 is the gated ("up")
    branch and W2 projects back to the model width.  All stored [out, in]."""
    A = X @ _weight(w, "W1").T
    G = X @ _weight(w, "W3").T
    H = silu(A) * G
    return H @ _weight(w, "W2").T


def _expert_fn(kind: str):
    return expert_linear_bias if kind == "linear_bias" else expert_swiglu


# ---------------------------------------------------------------- layer
def forward(x, W_g, b_g, k, E, expert, *, kind="swiglu", C=-1, shared=None,
            idx_override=None, logits=None, overflow="drop", rounds=0, groups=0,
            topk_groups=0):
    """The whole layer, masked loop over experts (tutorial §3.1).

    expert(e) -> dict of that expert's weights; shared() -> dict or None.
    idx_override replaces the oracle's own top-k selection (used when a token's
    top-k margin is too small for the selection to be unique in fp32); the
    weights are then those of the given selection.

    overflow: "drop" (dropped assignments add nothing), "reroute" (reroute()
    with `rounds` rounds; an assignment keeps its weight at its new expert)
    or "shared" (the dropped weights are added to the shared expert's weight
    of 1).  groups / topk_groups: group-limited routing (route()); not
    combined with re-routing.

    Returns a dict with logits, idx, w, final (the expert each assignment
    ends at, -1 dropped), the dispatch fields of `final` and y[T, d]
    (float64; the MoE branch only: the residual is the caller's)."""
    if logits is None:
        logits = router_logits(x, W_g, b_g)
    if idx_override is None:
        idx, w = route(logits, k, groups, topk_groups)
    else:
        idx = np.asarray(idx_override, dtype=np.int32)
        w = weights_for(logits, idx)
    final = _final_assignment(logits, idx, E, C, overflow, rounds, groups)
    dsp = dispatch(final, w, E, -1)
    dsp["counts"] = bincount(idx, E)  # the router's loads, before capacity
    dsp["C"] = C
    X = widen(x)
    T, d = X.shape
    y = np.zeros((T, d), dtype=np.float64)
    f = _expert_fn(kind)
    for e in range(E):
        mask = final == e
        t_rows, j_rows = np.nonzero(mask)
        if t_rows.size == 0:
            continue
        Y = f(X[t_rows], expert(e))
        y[t_rows] += w[t_rows, j_rows][:, None] * Y  # a token reaches e at most once
    if shared is not None:
        sw = shared()
        if sw is not None:
            y += _shared_weight(w, final, overflow)[:, None] * expert_swiglu(X, sw)
    out = dict(logits=logits, idx=idx, w=w, final=final, y=y)
    out.update(dsp)
    return out


def _final_assignment(logits, idx, E, C, overflow, rounds, groups=0):
    """The expert each (token, slot) ends at under the overflow policy."""
    if overflow == "reroute":
        if groups > 1:
            raise ValueError("re-routing is not defined with group-limited routing")
        return reroute(logits, idx, E, C, rounds)
    if overflow not in ("drop", "shared"):
        raise ValueError(f"overflow policy {overflow!r}")
    if C < 0:
        return np.asarray(idx, dtype=np.int64).copy()
    return np.where(capacity_ranks(idx, E) < C, idx, -1).astype(np.int64)


def _shared_weight(w, final, overflow):
    """Weight of the shared expert per token: 1, plus the dropped assignments'
    weights under the "shared" policy (tutorial Q2)."""
    sw = np.ones(w.shape[0], dtype=np.float64)
    if overflow == "shared":
        sw += np.where(final < 0, w, 0.0).sum(axis=1)
    return sw


def forward_tokens(tokens, x, W_g, b_g, k, E, expert, *, kind="swiglu", C=-1,
                   shared=None, idx_override=None, overflow="drop", rounds=0, logits=None,
                   groups=0, topk_groups=0):
    """The same layer evaluated only at the given tokens.

    Routing, counts and capacity ranks are computed for all T tokens (a
    token's drop depends on every earlier token), the expert evaluation only
    for the requested rows.  Experts are visited one at a time so each
    expert's weights are widened once.  Returns (y_rows [len(tokens), d],
    full routing/dispatch dict).  logits: as in forward()."""
    if logits is None:
        logits = router_logits(x, W_g, b_g)
    if idx_override is None:
        idx, w = route(logits, k, groups, topk_groups)
    else:
        idx = np.asarray(idx_override, dtype=np.int32)
        w = weights_for(logits, idx)
    final = _final_assignment(logits, idx, E, C, overflow, rounds, groups)
    dsp = dispatch(final, w, E, -1)
    dsp["counts"] = bincount(idx, E)
    dsp["C"] = C
    tokens = np.asarray(tokens, dtype=np.int64)
    X = widen(x[tokens])
    y = np.zeros((tokens.size, X.shape[1]), dtype=np.float64)
    f = _expert_fn(kind)
    sel_final = final[tokens]
    sel_w = w[tokens]
    for e in np.unique(sel_final[sel_final >= 0]):
        r, j = np.nonzero(sel_final == e)
        Y = f(X[r], expert(int(e)))
        y[r] += sel_w[r, j][:, None] * Y
    if shared is not None:
        sw = shared()
        if sw is not None:
            y += _shared_weight(sel_w, sel_final, overflow)[:, None] * expert_swiglu(X, sw)
    out = dict(logits=logits, idx=idx, w=w, final=final)
    out.update(dsp)
    return y, out


def dense_forward(x, W_g, b_g, k, E, expert, *, kind="swiglu", C=-1, shared=None,
                  overflow="drop", rounds=0, groups=0, topk_groups=0):
    """Brute force for tiny inputs: run every expert on every token, then sum
    over all experts with a dense [T, E] weight that is w[t, j] where expert e
    is where token t's j-th choice ends (kept, or re-routed) and 0 elsewhere
    (the sum-over-all-experts form of the iopenshare §1.2 Switch layer,
    weighted); the shared expert's weight is 1 plus, under the "shared"
    policy, every weight left without an expert.  Must equal forward()."""
    logits = router_logits(x, W_g, b_g)
    idx, w = route(logits, k, groups, topk_groups)
    T = idx.shape[0]
    if overflow == "reroute":
        dest = reroute(logits, idx, E, C, rounds)
    else:
        rank = capacity_ranks(idx, E)
        dest = np.where((C < 0) | (rank < C), idx, -1)
    Wd = np.zeros((T, E), dtype=np.float64)
    Ws = np.ones(T, dtype=np.float64)
    for t in range(T):
        for j in range(k):
            if dest[t, j] >= 0:
                Wd[t, dest[t, j]] = w[t, j]
            elif overflow == "shared":
                Ws[t] += w[t, j]
    X = widen(x)
    f = _expert_fn(kind)
    y = np.zeros_like(X)
    for e in range(E):
        y += Wd[:, e:e + 1] * f(X, expert(e))
    if shared is not None:
        sw = shared()
        if sw is not None:
            y += Ws[:, None] * expert_swiglu(X, sw)
    return y
