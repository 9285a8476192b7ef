"""GPU parity of the overflow policies (re-routing past capacity, overflow to
the shared expert) against the oracle.

moe_reroute from given logits must equal oracle.reroute bit for bit; the
grouping of its result (moe_dispatch over -1 entries) must equal
oracle.dispatch; moe_forward under each policy must match oracle.forward
within the layer tolerances, with counts and offsets bit-exact.  End to end,
both sides take the routing decisions on the GPU's fp32 logits, which are
themselves checked against the oracle's float64 logits.
"""
import json
import os

import numpy as np
import pytest

import oracle
from moe_synth import Workload, custom_config, get_config
from tests.conftest import GOLDEN
from tests.parity import ExpertStream, expert_bytes_f64
from tests.parity import check_forward, gpu_forward, gpu_logits, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_bincount_amd as m
    return m


def _gpu_reroute(moe, logits, idx, E, C, rounds):
    T, k = idx.shape
    s = moe.make_shape(T, 256, E, k, capacity=C, reroute_rounds=rounds)
    fin = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    moe.moe_reroute(s, torch.from_numpy(np.ascontiguousarray(logits)).cuda(),
                    torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda(), fin,
                    moe.workspace(s))
    torch.cuda.synchronize()
    return fin.cpu().numpy()


def test_reroute_hand_worked_examples(moe):
    with open(os.path.join(GOLDEN, "reroute_examples.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        print(f"[reroute golden] {c['name']}", flush=True)
        logits = np.array(c["logits"], np.float32)
        idx, _ = oracle.route(logits, c["k"])
        got = _gpu_reroute(moe, logits, idx, c["E"], c["C"], c["rounds"])
        assert got.tolist() == c["expected"], c["name"]


def _skewed_logits(T, E, seed, ties):
    rng = np.random.default_rng(seed)
    if ties:
        l = rng.integers(-4, 5, size=(T, E)).astype(np.float32)   # many exact ties
    else:
        l = rng.standard_normal((T, E)).astype(np.float32)
    l += np.log(1.0 / (np.arange(E) + 1.0)).astype(np.float32) * 1.5  # zipf-like skew
    return l


@pytest.mark.parametrize("T,E,k,C,rounds,ties", [
    (64, 4, 1, 10, 1, True),          # one chunk, k = 1
    (1000, 8, 2, 200, 1, True),       # two chunks
    (3000, 8, 2, 700, 3, False),      # six chunks, ragged tail
    (3000, 16, 4, 600, 2, True),
    (2000, 64, 2, 50, 5, True),       # most of the load re-routed
    (500, 256, 8, 12, 2, True),       # 256 experts, k = 8
    (129, 1024, 32, 3, 2, False),     # 1024 experts, k = 32 (KR = 96)
    (700, 6, 3, 300, 4, True),        # more rounds than E - k: capped at 3
    (1500, 24, 5, 220, 3, True),      # k = 5: chunks of 1020 assignments
    (2000, 12, 6, 800, 2, False),     # k = 6: chunks of 1020 assignments
    (400, 8, 2, 0, 3, False),         # C = 0: nothing placed
    (400, 8, 2, 100, 0, False),       # zero rounds: the capacity drop
    (300, 8, 2, -1, 2, True),         # unlimited capacity: unchanged
    (1, 4, 2, 0, 1, False)])
def test_reroute_bit_exact(moe, T, E, k, C, rounds, ties):
    print(f"[reroute] T={T} E={E} k={k} C={C} rounds={rounds} ties={ties}", flush=True)
    l = _skewed_logits(T, E, seed=T + 17 * E + k + rounds, ties=ties)
    idx, _ = oracle.route(l, k)
    got = _gpu_reroute(moe, l, idx, E, C, rounds)
    want = oracle.reroute(l, idx, E, C, rounds)
    assert np.array_equal(got, want), f"{(got != want).sum()} entries differ"


@pytest.mark.parametrize("T,E,k,C,rounds", [(1000, 8, 2, 180, 2), (2500, 64, 4, 120, 3)])
def test_dispatch_of_rerouted_selection(moe, T, E, k, C, rounds):
    """moe_dispatch over the final experts (-1 = no expert) groups exactly
    what oracle.dispatch does with the same -1 entries."""
    print(f"[reroute dispatch] T={T} E={E} k={k} C={C} rounds={rounds}", flush=True)
    l = _skewed_logits(T, E, seed=5 * T + E, ties=True)
    idx, w = oracle.route(l, k)
    fin = oracle.reroute(l, idx, E, C, rounds)
    s = moe.make_shape(T, 256, E, k, capacity=C)
    ws = moe.workspace(s)
    A = T * k
    P_max = min(A, E * C)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    keep = torch.full((A,), 9, dtype=torch.uint8, device="cuda")
    perm_token = torch.empty(P_max, dtype=torch.int32, device="cuda")
    perm_w = torch.empty(P_max, dtype=torch.float32, device="cuda")
    slot_pos = torch.full((A,), -9, dtype=torch.int32, device="cuda")
    moe.moe_dispatch(s, torch.from_numpy(fin.astype(np.int32)).cuda(),
                     torch.from_numpy(w.astype(np.float32)).cuda(), None, counts, offsets, keep,
                     perm_token, perm_w, slot_pos, None, ws)
    torch.cuda.synchronize()
    r = oracle.dispatch(fin, w, E, C)
    P = int(r["offsets"][-1])
    assert np.array_equal(counts.cpu().numpy(), r["counts"])
    assert np.array_equal(offsets.cpu().numpy(), r["offsets"])
    assert np.array_equal(keep.cpu().numpy().astype(bool), r["keep"].ravel())
    assert np.array_equal(slot_pos.cpu().numpy(), r["slot_pos"].ravel())
    assert np.array_equal(perm_token.cpu().numpy()[:P], r["perm_token"])
    np.testing.assert_array_equal(perm_w.cpu().numpy()[:P], r["perm_w"].astype(np.float32))


# T, d, E, k, d_ff, cf, shared, w, bias, overflow, rounds, combine
FORWARD = [
    (1000, 256, 8, 2, 256, 1.0, False, "bf16", "zipf1.5", "reroute", 1, None),
    (1000, 256, 8, 2, 256, 1.0, False, "bf16", "zipf1.5", "reroute", 6, None),
    (777, 512, 16, 4, 128, 0.75, True, "bf16", "zipf1.5", "reroute", 2, "grouped"),
    (777, 512, 16, 4, 128, 0.75, True, "bf16", "zipf1.5", "reroute", 2, "fused"),
    (96, 256, 16, 2, 384, 0.75, True, "fp8_e4m3", "zipf1.5", "reroute", 3, None),
    (600, 256, 8, 2, 256, 1.0, True, "bf16", "zipf1.5", "shared", 0, "grouped"),
    (600, 256, 8, 2, 256, 1.0, True, "bf16", "zipf1.5", "shared", 0, "fused"),
    (64, 512, 8, 2, 1408, 0.5, True, "fp8_e4m3", "zipf1.5", "shared", 0, None),
    (300, 256, 4, 2, 256, None, True, "bf16", None, "shared", 0, None),   # nothing dropped
]


@pytest.mark.parametrize("T,d,E,k,d_ff,cf,shared,w,bias,overflow,rounds,combine", FORWARD)
def test_forward_overflow(moe, T, d, E, k, d_ff, cf, shared, w, bias, overflow,
                          rounds, combine):
    print(f"[forward {overflow}] T={T} d={d} E={E} k={k} d_ff={d_ff} cf={cf} shared={shared} "
          f"w={w} rounds={rounds} combine={combine}", flush=True)
    cfg = custom_config(T, d, E, k, d_ff, w=w, cf=cf, shared=shared, router_bias=bias,
                        seed=3 * T + d + E)
    wl = Workload(cfg)
    out, layer, dev = gpu_forward(wl, overflow=overflow, rounds=rounds, combine=combine or "auto")
    gl = gpu_logits(layer, dev)
    rep = check_forward(wl, out, overflow=overflow, rounds=rounds, decide_on=gl)
    # the policy matters here: the drop policy's result is measurably different
    if cf is not None:
        base = oracle.forward(wl.x(), wl.W_g(), wl.b_g(), k, E, wl.expert, C=rep["C"],
                              shared=wl.shared if shared else None,
                              logits=gl.astype(np.float64))
        assert rel_err(out["y"], base["y"]) > 10 * rep["err"]
    print(f"  err={rep['err']:.3e} kept={rep['kept']}", flush=True)


def test_staged_shared_overflow(moe):
    """moe_expert_ffn into a grouped output, then moe_combine under overflow
    to the shared expert, against moe_forward; the fused form of
    moe_expert_ffn refuses the policy."""
    cfg = custom_config(500, 256, 8, 2, 256, cf=1.0, shared=True, router_bias="zipf1.5", seed=91)
    wl = Workload(cfg)
    out, layer, dev = gpu_forward(wl, overflow="shared")
    s = layer.shape
    ws = moe.workspace(s)
    T, k, d, E = cfg.T, cfg.k, cfg.d, cfg.E
    A = T * k
    C = moe.moe_capacity(T, E, k, cfg.cf)
    P_max = min(A, E * C)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm_token = torch.empty(P_max, dtype=torch.int32, device="cuda")
    perm_w = torch.empty(P_max, dtype=torch.float32, device="cuda")
    slot_pos = torch.empty(A, dtype=torch.int32, device="cuda")
    moe.moe_dispatch(s, layer.topk_idx, layer.topk_w, None, counts, offsets, None, perm_token,
                     perm_w, slot_pos, None, ws)
    y_perm = torch.empty((P_max + T, d), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(s, layer.weights, dev["x"], offsets, perm_token, None, y_perm, None, ws)
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    moe.moe_combine(s, y_perm, slot_pos, layer.topk_w, y)
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), out["y"]) < 1e-5
    gl = gpu_logits(layer, dev)
    out2 = dict(out)
    out2["y"] = y.cpu().numpy()
    check_forward(wl, out2, overflow="shared", decide_on=gl)
    with pytest.raises(moe.MoEError, match="UNSUPPORTED"):
        moe.moe_expert_ffn(s, layer.weights, dev["x"], offsets, perm_token, perm_w, None, y, ws)


@pytest.mark.parametrize("rounds", [1, 4])
def test_capacity_skew_rerouted_full_size(moe, rounds):
    """The skewed workload (16384 tokens, 64 experts, C = 640) with its
    overflow re-routed, in the launch configuration the benchmark times,
    compared on every token."""
    print(f"[capacity_skew reroute] rounds={rounds}", flush=True)
    wl = Workload(get_config("capacity_skew"))
    host = {}
    out, layer, dev = gpu_forward(wl, overflow="reroute", rounds=rounds, keep_host=host)
    gl = gpu_logits(layer, dev)
    stream = ExpertStream(lambda e: host[e], wl.cfg.E, expert_bytes_f64(wl.cfg))
    try:
        rep = check_forward(wl, out, overflow="reroute", rounds=rounds, decide_on=gl,
                            experts=stream)
    finally:
        stream.close()
    assert rep["tokens"] == wl.cfg.T
    print(f"  err={rep['err']:.3e} (nonzero rows {rep['err_nonzero_rows']:.3e}) "
          f"kept={rep['kept']}", flush=True)
