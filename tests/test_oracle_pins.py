"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign or index, a transposed operand, a wrong tie rule) fails it.  No
expected value here comes from the HIP path.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import moe_oracle as mo
from tests.conftest import GOLDEN

pytestmark = pytest.mark.cpu


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ a2: routing
def test_renormalisation_page_example():
    g = _golden("renorm_example.json")
    p = np.array([g["probs"]])
    logits = np.log(p).astype(np.float32)          # softmax(log p) = p
    idx, w = oracle.route(logits, g["k"])
    assert idx.tolist() == [g["expected_idx"]]
    exact = [float(Fraction(s)) for s in g["expected_w_exact"]]
    np.testing.assert_allclose(w[0], exact, rtol=0, atol=1e-7)   # fp32 log rounding
    np.testing.assert_allclose(np.round(w[0], g["printed_decimals"]), g["expected_w_printed"])
    assert abs(w.sum() - 1.0) < 1e-15


def test_weights_sum_to_one_and_two_formulations_agree():
    rng = np.random.default_rng(1)
    for E, k in [(4, 2), (8, 2), (64, 2), (256, 8), (7, 7), (5, 1)]:
        logits = rng.standard_normal((50, E)).astype(np.float32) * 3
        idx, w = oracle.route(logits, k)
        idx2, w2 = oracle.route_softmax_of_topk(logits, k)
        assert np.array_equal(idx, idx2)
        np.testing.assert_allclose(w, w2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
        # weights follow the slot order (slot 0 = largest logit)
        assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_topk_matches_brute_force_and_tie_rule():
    rng = np.random.default_rng(2)
    # values from a small grid force many exact ties
    logits = rng.integers(-3, 4, size=(200, 9)).astype(np.float32)
    logits[0, :] = 0.0
    logits[0, 3] = -0.0          # -0.0 ties with +0.0
    for k in (1, 2, 5, 9):
        idx = oracle.select_topk(logits, k)
        for t in range(logits.shape[0]):
            ref = sorted(range(9), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert idx[t].tolist() == ref
    assert oracle.select_topk(logits[:1], 4)[0].tolist() == [0, 1, 2, 3]


def test_k1_is_switch_routing_weight_one():
    # iopenshare §1.2: Switch routing keeps a single expert (argmax); the
    # renormalised weight of one kept expert is 1.
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((100, 8)).astype(np.float32)
    idx, w = oracle.route(logits, 1)
    assert np.array_equal(idx[:, 0], np.argmax(logits, axis=1))
    assert np.all(w == 1.0)


def test_k_equals_E_is_soft_routing():
    # MOE 学习笔记, 路由策略: soft routing weights every expert by the router's
    # probability distribution; with k = E nothing is dropped by top-k.
    from scipy.special import softmax
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((30, 6)).astype(np.float32)
    idx, w = oracle.route(logits, 6)
    dense = np.zeros_like(w)
    np.put_along_axis(dense, idx.astype(np.int64), w, axis=1)
    np.testing.assert_allclose(dense, softmax(logits.astype(np.float64), axis=1), atol=1e-14)


def test_shift_invariance_safe_softmax():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((40, 8)) * 2
    a = oracle.route(logits, 2)
    b = oracle.route(logits + 1000.0, 2)   # would overflow exp without the max shift
    assert np.array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], atol=1e-9)


def test_router_logits_one_hot_closed_form():
    # x rows that are unit vectors pick out rows of W_g[d, E]; a transposed
    # W_g or a missing bias fails.
    d, E = 6, 4
    rng = np.random.default_rng(6)
    W_g = rng.standard_normal((d, E)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    x = np.eye(d, dtype=np.float32)
    np.testing.assert_array_equal(oracle.router_logits(x, W_g), W_g)
    np.testing.assert_allclose(oracle.router_logits(2 * x, W_g, b), 2 * W_g + b, rtol=1e-7)


def test_bf16_widening_definition():
    # bfloat16 is the upper half of an IEEE binary32: 0x3F80 = 1.0,
    # 0xC000 = -2.0, 0x3F81 = 1 + 2^-7, 0x0001 = 2^-133 (subnormal).
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F], dtype=np.uint16)
    v = oracle.widen(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 1 + 2.0 ** -7
    assert v[3] == 2.0 ** -133
    assert v[4] == (2 - 2.0 ** -7) * 2.0 ** 127


# ------------------------------------------------------------------ a3: bincount / capacity
def test_bincount_sums_to_T_times_k_and_brute_force():
    g = _golden("lpt_example.json")
    assert sum(g["load"]) == g["total_routings"] == g["T"] * g["k"]
    rng = np.random.default_rng(7)
    for T, E, k in [(64, 4, 2), (300, 16, 3), (1, 8, 8)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        idx, _ = oracle.route(logits, k)
        c = oracle.bincount(idx, E)
        assert c.sum() == T * k
        assert [sum(1 for t in range(T) for j in range(k) if idx[t, j] == e) for e in range(E)] == c.tolist()


def test_capacity_definition_bounds():
    for T, E, k, cf in [(16384, 64, 2, 1.25), (64, 4, 2, 1.25), (4096, 8, 2, 1.0),
                        (1000, 7, 3, 1.1), (5, 256, 8, 2.0), (64, 4, 2, 0.3125)]:
        C = oracle.capacity(T, E, k, cf)
        # C*E/(T*k) is the realised capacity factor: at least cf, less than one
        # token per expert above it.
        assert Fraction(C * E, T * k) >= Fraction(cf)
        assert Fraction(C * E, T * k) < Fraction(cf) + Fraction(E, T * k)
    assert oracle.capacity(16384, 64, 2, 1.25) == 640
    assert oracle.capacity(64, 4, 2, None) == -1
    assert oracle.capacity(64, 4, 2, 0.0) == -1


def _idx_with_loads(loads, k, rng):
    """A [T, k] selection whose bincount is `loads` (each token picks k
    distinct experts).  Greedy on the largest remaining loads."""
    loads = list(loads)
    T = sum(loads) // k
    rows = []
    for _ in range(T):
        order = sorted(range(len(loads)), key=lambda e: (-loads[e], e))[:k]
        for e in order:
            loads[e] -= 1
        rows.append(order)
    assert all(v == 0 for v in loads)
    idx = np.array(rows, dtype=np.int32)
    return idx[rng.permutation(T)]


def test_capacity_drop_page_example():
    g = _golden("capacity_example.json")
    rng = np.random.default_rng(8)
    idx = _idx_with_loads(g["load"], 2, rng)
    w = np.full(idx.shape, 0.5)
    r = oracle.dispatch(idx, w, 4, g["capacity"])
    assert r["kept"].tolist() == g["expected_kept"]
    assert int(r["counts"][0] - r["kept"][0]) == g["expected_overflow_expert0"]
    # dropped in token order: expert 0's kept tokens are its first 20 tokens
    toks0 = [t for t in range(idx.shape[0]) if 0 in idx[t]]
    kept0 = sorted(int(r["perm_token"][p]) for p in range(r["offsets"][0], r["offsets"][1]))
    assert kept0 == toks0[:20]


def test_capacity_large_equals_unlimited_and_zero_drops_all():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((100, 8)).astype(np.float32)
    idx, w = oracle.route(logits, 2)
    a = oracle.dispatch(idx, w, 8, -1)
    b = oracle.dispatch(idx, w, 8, int(a["counts"].max()))
    for key in ("kept", "offsets", "perm_token", "slot_pos"):
        assert np.array_equal(a[key], b[key])
    z = oracle.dispatch(idx, w, 8, 0)
    assert z["offsets"][-1] == 0 and not z["keep"].any()


# ------------------------------------------------------------------ a4: permutation
def test_dispatch_permutation_invariants():
    rng = np.random.default_rng(10)
    for T, E, k, C in [(200, 8, 2, -1), (200, 8, 2, 30), (77, 5, 3, 20), (64, 4, 2, 20)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        logits[:, 0] += 1.0  # skew so the capacity binds
        idx, w = oracle.route(logits, k)
        r = oracle.dispatch(idx, w, E, C)
        P = r["offsets"][-1]
        # a bijection between kept (t, j) and positions 0..P-1
        kept_pairs = {(t, j) for t in range(T) for j in range(k) if r["keep"][t, j]}
        assert len(kept_pairs) == P
        seen = set()
        for p in range(P):
            t, j = int(r["perm_token"][p]), int(r["perm_slot"][p])
            assert (t, j) in kept_pairs and r["slot_pos"][t, j] == p
            seen.add((t, j))
            assert r["perm_w"][p] == w[t, j]
        assert seen == kept_pairs
        # sorted by (expert, token)
        keys = [(int(idx[r["perm_token"][p], r["perm_slot"][p]]), int(r["perm_token"][p])) for p in range(P)]
        assert keys == sorted(keys)
        # segment e holds exactly expert e's kept assignments
        for e in range(E):
            seg = range(r["offsets"][e], r["offsets"][e + 1])
            assert all(idx[r["perm_token"][p], r["perm_slot"][p]] == e for p in seg)
        assert np.all(r["slot_pos"][~r["keep"]] == -1)


# ------------------------------------------------------------------ a5/a6/a8: experts and combine
def test_silu_and_swiglu_closed_form():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(np.array([1.0, -1.0, 2.0])),
                               [1 / (1 + math.exp(-1)), -1 / (1 + math.exp(1)), 2 / (1 + math.exp(-2))],
                               rtol=1e-15)
    d = 3
    I = np.eye(d, dtype=np.float32)
    w = {"W1": I, "W3": 2 * I, "W2": I}
    X = np.array([[1.0, -1.0, 0.5]])
    Y = oracle.expert_swiglu(X, w)
    # silu applies to the W1 product, the W3 product is the linear gate
    ref = oracle.silu(X) * (2 * X)
    np.testing.assert_allclose(Y, ref, rtol=1e-15)
    assert not np.allclose(Y, oracle.silu(2 * X) * X)
    # W2 maps d_ff back to d and is stored [out, in]
    W2 = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=np.float32)
    Y2 = oracle.expert_swiglu(X, {"W1": I, "W3": 2 * I, "W2": W2})
    np.testing.assert_allclose(Y2[0], ref[0][[1, 2, 0]], rtol=1e-15)


def test_linear_bias_expert_closed_form():
    W = np.array([[1, 2], [3, 4]], dtype=np.float32)    # [out, in]
    b = np.array([0.5, -0.5], dtype=np.float32)
    Y = oracle.expert_linear_bias(np.array([[1.0, 0.0], [0.0, 1.0]]), {"W": W, "b": b})
    np.testing.assert_allclose(Y, [[1.5, 2.5], [2.5, 3.5]])


def test_combine_page_example():
    g = _golden("combine_example.json")
    outs = np.array(g["expert_outputs"], dtype=np.float32)
    wts = g["weights"]
    # two experts whose output ignores x (W = 0, bias = the printed output)
    experts = [{"W": np.zeros((2, 2), np.float32), "b": outs[e]} for e in range(2)]
    W_g = np.zeros((2, 2), np.float32)
    b_g = np.log(np.array(wts)).astype(np.float32)   # softmax(b_g) = (0.7, 0.3)
    x = np.ones((1, 2), np.float32)
    r = oracle.forward(x, W_g, b_g, 2, 2, lambda e: experts[e], kind="linear_bias")
    np.testing.assert_allclose(r["y"][0], g["expected"], atol=1e-7)
    # swapping which weight goes with which expert would give [0.41, 0.33]
    assert abs(r["y"][0, 0] - 0.41) > 0.1


def _tiny_swiglu(T, d, E, d_ff, seed, shared=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    W_g = (rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    ex = [{"W1": (rng.standard_normal((d_ff, d)) / np.sqrt(d)).astype(np.float32),
           "W3": (rng.standard_normal((d_ff, d)) / np.sqrt(d)).astype(np.float32),
           "W2": (rng.standard_normal((d, d_ff)) / np.sqrt(d_ff)).astype(np.float32)}
          for _ in range(E)]
    sh = None
    if shared:
        sh = {"W1": (rng.standard_normal((d_ff, d)) / np.sqrt(d)).astype(np.float32),
              "W3": (rng.standard_normal((d_ff, d)) / np.sqrt(d)).astype(np.float32),
              "W2": (rng.standard_normal((d, d_ff)) / np.sqrt(d_ff)).astype(np.float32)}
    return x, W_g, ex, sh


@pytest.mark.parametrize("T,d,E,k,d_ff,C,shared", [
    (40, 8, 4, 2, 12, -1, False), (40, 8, 4, 2, 12, 9, False),
    (33, 6, 8, 3, 10, 7, True), (20, 5, 6, 6, 4, -1, False), (25, 4, 5, 1, 3, 4, True)])
def test_masked_loop_equals_dense_brute_force(T, d, E, k, d_ff, C, shared):
    x, W_g, ex, sh = _tiny_swiglu(T, d, E, d_ff, seed=T * 7 + E, shared=shared)
    shf = (lambda: sh) if shared else None
    r = oracle.forward(x, W_g, None, k, E, lambda e: ex[e], C=C, shared=shf)
    yd = oracle.dense_forward(x, W_g, None, k, E, lambda e: ex[e], C=C, shared=shf)
    np.testing.assert_allclose(r["y"], yd, rtol=0, atol=1e-12)


def test_identical_experts_give_the_expert_itself():
    # weights of a token sum to 1, so with identical experts y = expert(x)
    x, W_g, ex, _ = _tiny_swiglu(50, 8, 6, 16, seed=11)
    r = oracle.forward(x, W_g, None, 3, 6, lambda e: ex[0])
    np.testing.assert_allclose(r["y"], oracle.expert_swiglu(x.astype(np.float64), ex[0]), atol=1e-12)


def test_token_permutation_equivariance_and_expert_relabelling():
    x, W_g, ex, _ = _tiny_swiglu(30, 8, 5, 12, seed=12)
    base = oracle.forward(x, W_g, None, 2, 5, lambda e: ex[e])["y"]
    perm = np.random.default_rng(0).permutation(30)
    yp = oracle.forward(x[perm], W_g, None, 2, 5, lambda e: ex[e])["y"]
    np.testing.assert_allclose(yp, base[perm], atol=1e-12)
    rel = np.array([3, 0, 4, 1, 2])                # new expert e' = rel[e]
    inv = np.argsort(rel)
    W_g2 = np.empty_like(W_g)
    W_g2[:, rel] = W_g
    y2 = oracle.forward(x, W_g2, None, 2, 5, lambda e: ex[inv[e]])["y"]
    np.testing.assert_allclose(y2, base, atol=1e-12)


def test_capacity_zero_leaves_only_the_shared_expert():
    x, W_g, ex, sh = _tiny_swiglu(20, 8, 4, 8, seed=13, shared=True)
    r = oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], C=0, shared=lambda: sh)
    np.testing.assert_allclose(r["y"], oracle.expert_swiglu(x.astype(np.float64), sh), atol=1e-14)
    r0 = oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], C=0)
    assert np.all(r0["y"] == 0)


def test_forward_tokens_equals_forward():
    x, W_g, ex, sh = _tiny_swiglu(60, 8, 6, 8, seed=14, shared=True)
    b = np.linspace(0, -3, 6).astype(np.float32)
    full = oracle.forward(x, W_g, b, 2, 6, lambda e: ex[e], C=15, shared=lambda: sh)
    toks = [0, 5, 59, 33]
    yr, _ = oracle.forward_tokens(toks, x, W_g, b, 2, 6, lambda e: ex[e], C=15, shared=lambda: sh)
    np.testing.assert_allclose(yr, full["y"][toks], atol=1e-13)


def test_idx_override_recomputes_weights_and_capacity():
    x, W_g, ex, _ = _tiny_swiglu(30, 8, 4, 8, seed=15)
    r = oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], C=8)
    o = oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], C=8, idx_override=r["idx"])
    np.testing.assert_allclose(o["y"], r["y"], atol=0)
    alt = r["idx"].copy()
    alt[0] = alt[0][::-1]                       # swap slot order: same set, same y
    o2 = oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], C=8, idx_override=alt)
    np.testing.assert_allclose(o2["y"], r["y"], atol=1e-14)


def test_topk_margin():
    l = np.array([[3.0, 1.0, 2.0, 0.5]], np.float32)
    assert oracle.topk_margin(l, 1)[0] == 1.0          # 3 - 2
    assert oracle.topk_margin(l, 2)[0] == 1.0          # min(1, 1)
    assert oracle.topk_margin(l, 3)[0] == 0.5          # min(1, 1, 0.5)
    assert oracle.topk_margin(l, 4)[0] == 0.5          # k = E: last gap skipped


# ------------------------------------------------------------------ f3: replication + placement
def test_eplb_hand_worked_examples():
    g = _golden("eplb_replication_examples.json")
    for c in g["cases"]:
        p = oracle.eplb_plan(c["load"], c["devices"], c["extra"])
        assert p["replicas"].tolist() == c["replicas"], c["name"]
        assert p["slot_load"].tolist() == c["slot_load"], c["name"]
        assert p["slot_device"].tolist() == c["slot_device"], c["name"]
        assert p["device_load"].tolist() == c["device_load"], c["name"]
        p0 = oracle.eplb_plan(c["load"], c["devices"], 0)
        assert p0["device_load"].tolist() == c["device_load_without_replicas"], c["name"]


def test_eplb_without_replicas_is_the_tutorial_lpt():
    g = _golden("lpt_example.json")
    p = oracle.eplb_plan(g["load"], g["devices"], 0)
    assert p["slot_device"].tolist() == g["lpt_assignment"]
    assert p["device_load"].tolist() == g["lpt_device_load"]
    rng = np.random.default_rng(61)
    for E, D in [(8, 3), (64, 8), (256, 8), (5, 7)]:
        load = rng.integers(0, 400, size=E)
        load[rng.integers(0, E)] = 0
        a, dev = oracle.lpt_pack(load, D)
        p = oracle.eplb_plan(load, D, 0)
        assert np.array_equal(p["slot_device"], a) and np.array_equal(p["device_load"], dev)


def _dhondt(load, D, extra):
    """The replication stated as a highest-quotient apportionment: the extra
    replicas are the `extra` largest quotients load_e / j (j = 1 .. D-1, the
    quotient that earns replica j + 1), ordered by (-quotient, expert, j)."""
    from fractions import Fraction
    q = sorted(((Fraction(int(l), j), e, j) for e, l in enumerate(load) for j in range(1, D)),
               key=lambda v: (-v[0], v[1], v[2]))
    r = [1] * len(load)
    for _, e, _ in q[:extra]:
        r[e] += 1
    return r


@pytest.mark.parametrize("E,D,extra", [(8, 4, 3), (64, 8, 16), (256, 8, 32), (16, 2, 40),
                                       (6, 3, 20), (32, 8, 0)])
def test_eplb_replication_and_placement_invariants(E, D, extra):
    rng = np.random.default_rng(E * 7 + D + extra)
    load = (rng.zipf(1.6, size=E) * 10).clip(0, 5000)
    load[rng.integers(0, E)] = 0
    p = oracle.eplb_plan(load, D, extra)
    r = p["replicas"]
    assert r.tolist() == _dhondt(load, D, extra)
    assert r.sum() == E + min(extra, E * (D - 1)) and r.max() <= D
    # every expert's tokens are split over its replicas, evenly
    for e in range(E):
        sl = p["slot_load"][p["slot_expert"] == e]
        assert sl.sum() == load[e] and sl.max() - sl.min() <= 1
        devs = p["slot_device"][p["slot_expert"] == e]
        assert len(set(devs.tolist())) == devs.size      # copies on distinct devices
    assert p["device_load"].sum() == load.sum()
    for d in range(D):
        assert p["device_load"][d] == p["slot_load"][p["slot_device"] == d].sum()


# ------------------------------------------------------------------ f4: group-limited routing
def test_group_routing_hand_worked_examples():
    g = _golden("group_routing_examples.json")
    for c in g["cases"]:
        l = np.array([c["logits"]], np.float32)
        mask = oracle.select_groups(l, c["groups"], c["topk_groups"])
        assert np.nonzero(mask[0])[0].tolist() == c["expected_groups"], c["name"]
        idx, w = oracle.route(l, c["k"], c["groups"], c["topk_groups"])
        assert idx[0].tolist() == c["expected_idx"], c["name"]
        assert oracle.route(l, c["k"])[0][0].tolist() == c["expected_idx_without_groups"]
        # the weights follow the ungrouped rule on the chosen experts
        sel = l[0, idx[0]].astype(np.float64)
        np.testing.assert_allclose(w[0], np.exp(sel) / np.exp(sel).sum(), rtol=1e-12)


def test_group_routing_special_cases_reduce_to_plain_routing():
    rng = np.random.default_rng(51)
    for E, G, k in [(8, 4, 2), (16, 4, 3), (64, 8, 8), (12, 3, 5)]:
        l = rng.integers(-3, 4, size=(200, E)).astype(np.float32)   # many ties
        plain = oracle.route(l, k)[0]
        # keeping every group is plain routing
        assert np.array_equal(oracle.route(l, k, G, G)[0], plain)
        # one expert per group, keep k groups: the groups are the experts
        assert np.array_equal(oracle.route(l, k, E, k)[0], plain)


def test_group_routing_brute_force_order_and_limit():
    rng = np.random.default_rng(52)
    T, E, G, M, k = 300, 16, 8, 3, 4
    l = rng.integers(-4, 5, size=(T, E)).astype(np.float32)
    mask = oracle.select_groups(l, G, M)
    idx, w = oracle.route(l, k, G, M)
    gs = E // G
    for t in range(T):
        score = [max(float(v) for v in l[t, g * gs:(g + 1) * gs]) for g in range(G)]
        kept = [g for g in range(G) if mask[t, g]]
        assert len(kept) == M
        # every kept group is at least as good as every dropped one; equal
        # scores are kept in index order
        for g in kept:
            for h in range(G):
                if not mask[t, h]:
                    assert score[g] > score[h] or (score[g] == score[h] and g < h)
        # the experts lie in kept groups, and they are the best k of those
        assert all(mask[t, e // gs] for e in idx[t])
        allowed = sorted((e for e in range(E) if mask[t, e // gs]),
                         key=lambda e: (-float(l[t, e]), e))
        assert idx[t].tolist() == allowed[:k]
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)


def test_grouped_forward_equals_dense_brute_force():
    x, W_g, ex, sh = _tiny_swiglu(40, 8, 8, 12, seed=53, shared=True)
    kw = dict(C=9, shared=lambda: sh, groups=4, topk_groups=2)
    r = oracle.forward(x, W_g, None, 3, 8, lambda e: ex[e], **kw)
    yd = oracle.dense_forward(x, W_g, None, 3, 8, lambda e: ex[e], **kw)
    np.testing.assert_allclose(r["y"], yd, rtol=0, atol=1e-12)
    groups_used = {(t, int(e) // 2) for t in range(40) for e in r["idx"][t]}
    assert all(sum(1 for (t2, _) in groups_used if t2 == t) <= 2 for t in range(40))
    with pytest.raises(ValueError):
        oracle.forward(x, W_g, None, 3, 8, lambda e: ex[e], C=9, overflow="reroute", rounds=1,
                       groups=4, topk_groups=2)


# ------------------------------------------------------------------ f1: overflow policies
def test_reroute_hand_worked_examples():
    g = _golden("reroute_examples.json")
    for c in g["cases"]:
        logits = np.array(c["logits"], np.float32)
        idx, _ = oracle.route(logits, c["k"])
        got = oracle.reroute(logits, idx, c["E"], c["C"], c["rounds"])
        assert got.tolist() == c["expected"], c["name"]


def _reroute_by_queues(logits, idx, E, C, rounds):
    """The same re-routing stated per expert: each round every expert takes the
    queue of requests addressed to it, ordered by (token, slot), and admits the
    head of the queue up to its free room.  Preference lists come from a plain
    Python sort on (-logit, expert)."""
    T, k = idx.shape
    pref = [sorted(range(E), key=lambda e: (-float(logits[t, e]), e)) for t in range(T)]
    dest = {}
    room = {e: C for e in range(E)}
    for e in range(E):
        queue = sorted((t, j) for t in range(T) for j in range(k) if idx[t, j] == e)
        for t, j in queue[:C]:
            dest[(t, j)] = e
        room[e] = C - min(C, len(queue))
    asked = {t: set(int(v) for v in idx[t]) for t in range(T)}
    for _ in range(rounds):
        queues = {e: [] for e in range(E)}
        for t in range(T):
            for j in range(k):
                if (t, j) in dest:
                    continue
                left = [e for e in pref[t] if e not in asked[t]]
                if left:
                    asked[t].add(left[0])
                    queues[left[0]].append((t, j))
        for e, q in queues.items():
            for t, j in sorted(q)[:room[e]]:
                dest[(t, j)] = e
            room[e] -= min(room[e], len(q))
    return np.array([[dest.get((t, j), -1) for j in range(k)] for t in range(T)])


@pytest.mark.parametrize("T,E,k,C,rounds,skew", [
    (40, 4, 1, 8, 1, 1.5), (40, 4, 1, 8, 3, 1.5), (60, 8, 2, 10, 2, 2.0),
    (50, 6, 3, 20, 4, 1.0), (30, 5, 2, 3, 5, 3.0), (64, 16, 4, 12, 2, 2.5)])
def test_reroute_equals_queue_restatement_and_invariants(T, E, k, C, rounds, skew):
    rng = np.random.default_rng(T * 31 + E * 7 + rounds)
    logits = rng.integers(-4, 5, size=(T, E)).astype(np.float32)   # many ties
    logits[:, 0] += skew
    idx, _ = oracle.route(logits, k)
    fin = oracle.reroute(logits, idx, E, C, rounds)
    assert np.array_equal(fin, _reroute_by_queues(logits, idx, E, C, rounds))
    # capacity respected, experts distinct per token, first-pass keeps unchanged
    assert np.all(np.bincount(fin[fin >= 0], minlength=E) <= C)
    for t in range(T):
        got = fin[t][fin[t] >= 0]
        assert len(set(got.tolist())) == got.size
    first = oracle.dispatch(idx, np.ones(idx.shape), E, C)["keep"]
    assert np.array_equal(fin[first], idx[first])
    # a moved slot lands on an expert outside the token's own top-k
    moved = (fin >= 0) & ~first
    for t, j in zip(*np.nonzero(moved)):
        assert fin[t, j] not in idx[t]
    # more rounds only add: every placement of `rounds` survives in `rounds + 1`
    more = oracle.reroute(logits, idx, E, C, rounds + 1)
    assert np.all(more[fin >= 0] == fin[fin >= 0])
    assert (more >= 0).sum() >= (fin >= 0).sum()


def test_reroute_closed_forms():
    rng = np.random.default_rng(41)
    logits = rng.standard_normal((80, 8)).astype(np.float32)
    logits[:, 2] += 2.0
    idx, _ = oracle.route(logits, 2)
    C = 12
    drop = oracle.dispatch(idx, np.ones(idx.shape), 8, C)["keep"]
    assert np.array_equal(oracle.reroute(logits, idx, 8, C, 0), np.where(drop, idx, -1))
    big = int(np.bincount(idx.ravel()).max())
    assert np.array_equal(oracle.reroute(logits, idx, 8, big, 3), idx)
    assert np.array_equal(oracle.reroute(logits, idx, 8, -1, 3), idx)
    # C = 0: nothing can be placed however many rounds
    assert np.all(oracle.reroute(logits, idx, 8, 0, 6) == -1)
    # enough rounds: a slot stays dropped only if every expert its token does
    # not hold is full
    fin = oracle.reroute(logits, idx, 8, C, 8 - 2)
    load = np.bincount(fin[fin >= 0], minlength=8)
    for t, j in zip(*np.nonzero(fin < 0)):
        others = [e for e in range(8) if e not in fin[t]]
        assert all(load[e] == C for e in others)
    # re-routing never loses a first-pass keep
    assert (fin >= 0).sum() >= drop.sum()


@pytest.mark.parametrize("overflow,rounds", [("drop", 0), ("reroute", 1), ("reroute", 3),
                                             ("shared", 0)])
@pytest.mark.parametrize("T,d,E,k,d_ff,C", [(40, 8, 4, 2, 12, 9), (33, 6, 8, 3, 10, 7),
                                            (25, 4, 5, 1, 3, 4)])
def test_overflow_policies_equal_dense_brute_force(overflow, rounds, T, d, E, k, d_ff, C):
    x, W_g, ex, sh = _tiny_swiglu(T, d, E, d_ff, seed=T * 5 + E, shared=True)
    b = np.linspace(1.0, -1.0, E).astype(np.float32)     # skew so the capacity binds
    kw = dict(C=C, shared=lambda: sh, overflow=overflow, rounds=rounds)
    r = oracle.forward(x, W_g, b, k, E, lambda e: ex[e], **kw)
    yd = oracle.dense_forward(x, W_g, b, k, E, lambda e: ex[e], **kw)
    np.testing.assert_allclose(r["y"], yd, rtol=0, atol=1e-12)
    toks = [0, T // 2, T - 1]
    yr, _ = oracle.forward_tokens(toks, x, W_g, b, k, E, lambda e: ex[e], **kw)
    np.testing.assert_allclose(yr, r["y"][toks], rtol=0, atol=1e-12)


def test_overflow_to_shared_closed_forms():
    x, W_g, ex, sh = _tiny_swiglu(20, 8, 4, 8, seed=13, shared=True)
    X = x.astype(np.float64)
    # C = 0: every routed weight goes to the shared expert, and they sum to 1
    r = oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], C=0, shared=lambda: sh,
                       overflow="shared")
    np.testing.assert_allclose(r["y"], 2.0 * oracle.expert_swiglu(X, sh), rtol=1e-14, atol=1e-14)
    # nothing dropped: the same as the plain layer
    a = oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], shared=lambda: sh, overflow="shared")
    b = oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], shared=lambda: sh)
    assert np.array_equal(a["y"], b["y"])
    # identical routed and shared experts: y = 2 * expert(x) whatever is dropped
    r2 = oracle.forward(x, W_g, None, 2, 4, lambda e: sh, C=3, shared=lambda: sh,
                        overflow="shared")
    np.testing.assert_allclose(r2["y"], 2.0 * oracle.expert_swiglu(X, sh), rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.forward(x, W_g, None, 2, 4, lambda e: ex[e], C=3, overflow="spill")


# ------------------------------------------------------------------ a9: load stats
def test_lpt_page_example():
    g = _golden("lpt_example.json")
    a, dev = oracle.lpt_pack(g["load"], g["devices"])
    assert a.tolist() == g["lpt_assignment"]
    assert dev.tolist() == g["lpt_device_load"]
    naive = oracle.naive_split(g["load"], g["devices"])
    assert naive.tolist() == g["naive_device_load"]
    assert oracle.sample_variance(naive) == g["naive_variance"]
    assert oracle.sample_variance(dev) == g["lpt_variance"]
    assert round(oracle.expert_imbalance(g["load"]), 3) == g["imbalance_printed"]
    assert max(dev) == g["optimum_max_load"]


def _opt_makespan(load, D):
    best = None
    for assign in itertools.product(range(D), repeat=len(load)):
        bins = [0] * D
        for e, dv in enumerate(assign):
            bins[dv] += load[e]
        m = max(bins)
        best = m if best is None else min(best, m)
    return best


def test_lpt_four_thirds_bound_against_brute_force():
    rng = np.random.default_rng(16)
    for _ in range(60):
        E = int(rng.integers(2, 9))
        D = int(rng.integers(2, 4))
        load = rng.integers(0, 50, size=E).tolist()
        _, dev = oracle.lpt_pack(load, D)
        assert sum(dev) == sum(load)
        opt = _opt_makespan(load, D)
        assert max(dev) <= Fraction(4, 3) * opt + 0   # classical LPT bound
    # a tight-ish instance of the bound: 2 machines, loads 3,3,2,2,2 -> LPT 7, OPT 6
    _, dev = oracle.lpt_pack([3, 3, 2, 2, 2], 2)
    assert max(dev) == 7 and _opt_makespan([3, 3, 2, 2, 2], 2) == 6


def test_imbalance_epsilon_guards_empty_expert():
    assert oracle.expert_imbalance([5, 0, 3]) == pytest.approx(5 / 1e-6)
    assert oracle.expert_imbalance([4, 4]) == pytest.approx(1.0, abs=1e-6)


# ------------------------------------------------------------------ fp8 e4m3
def test_e4m3_table_against_format_definition_and_torch():
    t = oracle.e4m3_decode_table()
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and math.copysign(1, t[0x80]) == -1
    finite = t[~np.isnan(t)]
    assert finite.max() == 448.0
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                  # monotone over positive codes
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both = ~np.isnan(t)
    assert np.array_equal(np.isnan(ref), ~both)
    assert np.array_equal(ref[both], t[both])


def test_dequant_rows_group_scaling():
    codes = np.full((256, 3), 0x38, dtype=np.uint8)        # all 1.0
    s = np.array([0.5, 4.0], np.float32)
    W = oracle.dequant_rows(codes, s)
    assert np.all(W[:128] == 0.5) and np.all(W[128:] == 4.0)


def test_int8_dequant_definition_and_torch():
    """weight = code * scale, one scale per 128 output rows; the codes are the
    two's-complement bytes (torch's int8 cast agrees), and the synthetic
    quantiser keeps |code| <= 127 with round-trip error <= scale / 2."""
    codes = np.array([[-127, -1, 0, 1, 127]] * 256, dtype=np.int8)
    s = np.array([0.25, 3.0], np.float32)
    W = oracle.dequant_int8_rows(codes, s)
    assert W[0].tolist() == [-31.75, -0.25, 0.0, 0.25, 31.75]
    assert W[200].tolist() == [-381.0, -3.0, 0.0, 3.0, 381.0]
    import torch
    allc = np.arange(-128, 128, dtype=np.int64).astype(np.int8).reshape(1, 256).repeat(128, 0)
    ref = torch.from_numpy(allc).to(torch.float64).numpy() * 0.5
    assert np.array_equal(oracle.dequant_int8_rows(allc, np.array([0.5], np.float32)), ref)
    from moe_synth.gen import _quant_int8_rows, f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(3)
    w = f32_to_bf16_bits(rng.standard_normal((256, 64)).astype(np.float32))
    q, sc = _quant_int8_rows(w)
    assert q.dtype == np.int8 and np.abs(q.astype(np.int32)).max() == 127
    back = oracle.dequant_int8_rows(q, sc)
    err = np.abs(back - bf16_bits_to_f32(w).astype(np.float64))
    assert np.all(err <= np.repeat(sc.astype(np.float64), 128)[:, None] / 2 * (1 + 1e-6))



def test_int4_dequant_hand_worked_bytes():
    """Packed int4, worked by hand: offset-binary codes (c = n + 8), the 8
    inputs of a group in 4 bytes, byte b holding input b (low nibble) and
    input b + 4 (high nibble).  Bytes 08 F9 17 80 hold c = 8, 9, 7, 0 | 0,
    15, 1, 8, i.e. n = 0, 1, -1, -8, -8, 7, -7, 0; rows 128.. take the second
    scale."""
    b = np.array([[0x08, 0xF9, 0x17, 0x80]] * 256, dtype=np.uint8).view(oracle.INT4X2)
    W = oracle.dequant_int4_rows(b, np.array([0.5, 2.0], np.float32))
    assert W.shape == (256, 8)
    assert W[0].tolist() == [0.0, 0.5, -0.5, -4.0, -4.0, 3.5, -3.5, 0.0]
    assert W[255].tolist() == [0.0, 2.0, -2.0, -16.0, -16.0, 14.0, -14.0, 0.0]


def test_int4_unpack_all_bytes_by_bits():
    """Every byte value at every position of a group: the codes read from the
    byte's bits (numpy's unpackbits, most significant first) minus 8."""
    # row r, byte 4g + b holds (4g + b + r) mod 256: every value at every
    # byte position of a group, over the four rows
    packed = ((np.arange(256)[None, :] + np.arange(4)[:, None]) % 256).astype(np.uint8)
    got = oracle.unpack_int4(packed.view(oracle.INT4X2))
    bits = np.unpackbits(packed[:, :, None], axis=2).astype(np.int64)   # [4, 256, 8]
    hi = bits[:, :, 0:4] @ np.array([8, 4, 2, 1]) - 8
    lo = bits[:, :, 4:8] @ np.array([8, 4, 2, 1]) - 8
    for r in range(4):
        for byte in range(256):
            g, bpos = divmod(byte, 4)
            assert got[r, 8 * g + bpos] == lo[r, byte]
            assert got[r, 8 * g + bpos + 4] == hi[r, byte]
    for bpos in range(4):
        assert sorted(packed[:, bpos::4].ravel().tolist()) == list(range(256))


def test_int4_reduces_to_int8_and_synthetic_round_trip():
    """Codes in [-7, 7] packed as int4 (by the definition, one nibble at a
    time) decode to the same weights as the same codes stored as int8; the
    synthetic quantiser keeps |code| <= 7 (7 reached in every group) with
    round-trip error <= scale / 2."""
    rng = np.random.default_rng(11)
    codes = rng.integers(-7, 8, size=(256, 64)).astype(np.int8)
    packed = np.zeros((256, 32), dtype=np.uint8)
    for r in range(256):
        for k in range(64):
            g, j = divmod(k, 8)
            byte = 4 * g + (j % 4)
            c = int(codes[r, k]) + 8
            packed[r, byte] |= c if j < 4 else c << 4
    s = np.array([0.125, 3.0], np.float32)
    assert np.array_equal(oracle.dequant_int4_rows(packed.view(oracle.INT4X2), s),
                          oracle.dequant_int8_rows(codes, s))
    from moe_synth.gen import _quant_int4_rows, f32_to_bf16_bits, bf16_bits_to_f32
    w = f32_to_bf16_bits(rng.standard_normal((256, 64)).astype(np.float32))
    q, sc = _quant_int4_rows(w)
    assert q.shape == (256, 32)
    c = oracle.unpack_int4(q)
    assert np.abs(c).max() == 7
    assert all(np.abs(c[g * 128:(g + 1) * 128]).max() == 7 for g in range(2))
    back = oracle.dequant_int4_rows(q, sc)
    err = np.abs(back - bf16_bits_to_f32(w).astype(np.float64))
    assert np.all(err <= np.repeat(sc.astype(np.float64), 128)[:, None] / 2 * (1 + 1e-6))
