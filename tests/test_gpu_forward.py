"""GPU parity of the whole layer forward pass (moe_forward) against the oracle.

Small shapes are compared on every output element; they span several tiles in
every GEMM dimension with ragged row tails.  The named workloads run at full
size, in the launch configuration the benchmark times, and are compared on
every token as well: the oracle's loop over experts is fed each expert's
weights decoded ahead on a thread pool (ExpertStream), so it does not wait
for input generation.
"""
import numpy as np
import pytest

import oracle
from moe_synth import Workload, custom_config, get_config
from moe_synth.gen import INT4X2
from tests.parity import (ExpertStream, check_forward, expert_bytes_f64, gpu_forward, gpu_logits,
                          rel_err)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_bincount_amd as m
    return m


SMALL = [
    # T, d, E, k, d_ff, cf, shared, w, bias
    (1000, 256, 4, 2, 384, None, False, "bf16", None),
    (777, 512, 8, 2, 256, 1.0, False, "bf16", "zipf1.5"),
    (300, 256, 16, 4, 128, None, True, "bf16", None),
    (1, 256, 8, 2, 128, None, False, "bf16", None),
    (129, 768, 32, 8, 256, 0.5, True, "bf16", None),
    (500, 256, 8, 2, 256, None, True, "fp8_e4m3", None),
    (64, 512, 8, 2, 1408, None, False, "bf16", None),
    # few rows per expert (mostly empty row tiles, per-wave granule counts):
    # fp8, a shared expert over all tokens, and a capacity limit
    (64, 512, 8, 2, 1408, None, False, "fp8_e4m3", None),
    (48, 256, 4, 2, 256, None, True, "bf16", None),
    (96, 256, 16, 2, 384, 0.75, True, "fp8_e4m3", "zipf1.5"),
    # fp8 weights with 256 or more rows per expert (the ping-pong kernel's
    # 256 x 256 tiles)
    (1100, 512, 8, 2, 384, None, True, "fp8_e4m3", None),
    (2000, 256, 4, 2, 256, 1.0, False, "fp8_e4m3", "zipf1.5"),
    # long down-projection K with few tiles per XCD: every tile is a split
    # tail tile summed by the fixup pass (grouped output), bf16 and fp8
    (600, 512, 4, 2, 4096, None, True, "bf16", None),
    (600, 512, 4, 2, 4096, None, False, "fp8_e4m3", None),
    # long gate/up K (d = 4096) with few tiles: every gate/up tile is split,
    # its gate and up partial sums finished (SwiGLU) by the fixup pass
    (300, 4096, 4, 2, 256, None, True, "bf16", None),
    (600, 4096, 4, 2, 256, None, False, "fp8_e4m3", None),
    # 8-bit weights with 33..255 rows per expert: the ping-pong kernel's
    # 128 x 512 tiles (ragged row tiles, a shared expert's partial tiles,
    # partial weight tiles in both projections, a long K)
    (300, 4096, 4, 2, 256, None, False, "fp8_e4m3", None),
    (700, 768, 8, 2, 384, None, True, "fp8_e4m3", None),
    (600, 512, 8, 2, 640, None, True, "int8", None),
    (160, 256, 4, 2, 256, 1.0, False, "int8", "zipf1.5"),
    # the largest expert counts: 512 and 1024 experts (16 expert blocks in
    # the router, 1024 segments in the GEMM schedule)
    (700, 256, 512, 4, 128, None, False, "bf16", None),
    (1500, 256, 1024, 8, 128, 1.0, True, "bf16", None),
    # degenerate routing: one expert (k = E = 1), every expert (k = E = 4)
    (200, 256, 1, 1, 256, None, False, "bf16", None),
    (150, 256, 4, 4, 128, 1.0, True, "bf16", None),
    # int8 weights: full tiles, few rows per expert (three-stage pipeline),
    # a shared expert, a capacity limit
    (1100, 512, 8, 2, 384, None, True, "int8", None),
    (64, 512, 8, 2, 1408, None, False, "int8", None),
    (96, 256, 16, 2, 384, 0.75, True, "int8", "zipf1.5"),
    (600, 512, 4, 2, 4096, None, False, "int8", None),
    # int4 weights (two codes per byte): the same shapes, so both pipeline
    # shapes (16-byte weight rows per 32-deep step, 32-byte per 64-deep),
    # split tail tiles and the shared expert are covered
    (1100, 512, 8, 2, 384, None, True, "int4", None),
    (64, 512, 8, 2, 1408, None, False, "int4", None),
    (96, 256, 16, 2, 384, 0.75, True, "int4", "zipf1.5"),
    (600, 512, 4, 2, 4096, None, False, "int4", None),
    (300, 4096, 4, 2, 256, None, True, "int4", None),
    # decode-sized batches whose skewed routing gives one expert more rows
    # than the small activation tiles hold (several row tiles per expert)
    (64, 256, 8, 2, 256, None, False, "bf16", "zipf1.5"),
    (96, 256, 8, 2, 256, None, True, "bf16", "zipf1.5"),
    (96, 256, 8, 2, 256, None, True, "fp8_e4m3", "zipf1.5"),
    (96, 256, 8, 2, 256, None, False, "int8", "zipf1.5"),
    (96, 256, 8, 2, 256, None, True, "int4", "zipf1.5"),
]


@pytest.mark.parametrize("T,d,E,k,d_ff,cf,shared,w,bias", SMALL)
def test_forward_small(moe, T, d, E, k, d_ff, cf, shared, w, bias):
    print(f"[forward] T={T} d={d} E={E} k={k} d_ff={d_ff} cf={cf} shared={shared} w={w}",
          flush=True)
    cfg = custom_config(T, d, E, k, d_ff, w=w, cf=cf, shared=shared, router_bias=bias,
                        seed=T + d + E)
    wl = Workload(cfg)
    out, _, _ = gpu_forward(wl)
    rep = check_forward(wl, out)
    print(f"  err={rep['err']:.3e} flipped={rep['flipped']} kept={rep['kept']}", flush=True)


@pytest.mark.parametrize("T,d,E,k,d_ff,cf,shared,w,bias", [
    (777, 512, 8, 2, 256, 1.0, False, "bf16", "zipf1.5"),
    (600, 512, 4, 2, 4096, None, True, "bf16", None),        # split tail tiles, fixup
    (300, 4096, 4, 2, 256, None, True, "bf16", None),        # gate/up fixup writes lo too
    (64, 512, 8, 2, 1408, None, False, "bf16", None),        # decode-sized, fused combine
    (500, 256, 8, 2, 256, None, True, "fp8_e4m3", None),
    (1100, 512, 8, 2, 384, None, True, "int4", None),
    (96, 256, 16, 2, 384, 0.75, True, "int8", "zipf1.5")])
def test_forward_hidden_split(moe, T, d, E, k, d_ff, cf, shared, w, bias):
    """The compensated hidden activation (hi + lo bf16 terms): the same
    routing, and y much closer to the oracle than with a bf16 hidden
    activation (whose rounding then dominates the error), in every weight
    format and pipeline shape."""
    print(f"[hidden split] T={T} d={d} E={E} k={k} d_ff={d_ff} cf={cf} shared={shared} w={w}",
          flush=True)
    base = custom_config(T, d, E, k, d_ff, w=w, cf=cf, shared=shared, router_bias=bias,
                         seed=T + d + E + 1)
    wl1 = Workload(base)
    out1, _, dev = gpu_forward(wl1)
    rep1 = check_forward(wl1, out1)
    wl2 = Workload(base.with_(hidden_split=True))
    out2, _, _ = gpu_forward(wl2, dev=dev)
    rep2 = check_forward(wl2, out2)
    assert np.array_equal(out1["idx"], out2["idx"]) and np.array_equal(out1["counts"], out2["counts"])
    print(f"  err bf16 h {rep1['err']:.3e}, compensated h {rep2['err']:.3e}", flush=True)
    if w == "bf16":
        assert rep2["err"] < rep1["err"] / 20


def test_tiny_page_layer(moe):
    """The tutorial-sized fp32 layer: 64 tokens, width 8, 4 Linear experts, top-2."""
    wl = Workload(get_config("tiny"))
    out, _, _ = gpu_forward(wl)
    rep = check_forward(wl, out)
    assert out["counts"].sum() == 128
    print(f"[tiny] err={rep['err']:.3e} load={out['counts'].tolist()}", flush=True)


@pytest.mark.parametrize("T,seed,shared", [(600, 5, False), (64, 6, False), (200, 7, True)])
def test_unfused_path_matches_fused(moe, T, seed, shared):
    """moe_expert_ffn into a grouped output, then moe_combine, against the
    fused scatter-add path and the oracle (600 tokens; 64, a few rows per
    expert; 200 with a shared expert, whose rows follow the grouped rows)."""
    cfg = custom_config(T, 256, 8, 2, 256, cf=1.0, seed=seed, shared=shared)
    wl = Workload(cfg)
    out, layer, dev = gpu_forward(wl, combine="fused")
    s = layer.shape
    ws = moe.workspace(s)
    T, k, d = cfg.T, cfg.k, cfg.d
    A = T * k
    C = moe.moe_capacity(cfg.T, cfg.E, cfg.k, cfg.cf)
    P_max = min(A, cfg.E * C)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    perm_token = torch.empty(P_max, dtype=torch.int32, device="cuda")
    perm_w = torch.empty(P_max, dtype=torch.float32, device="cuda")
    slot_pos = torch.empty(A, dtype=torch.int32, device="cuda")
    moe.moe_dispatch(s, layer.topk_idx, layer.topk_w, None, counts, offsets, None, perm_token,
                     perm_w, slot_pos, None, ws)
    y_perm = torch.empty((P_max + (T if shared else 0), d), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(s, layer.weights, dev["x"], offsets, perm_token, None, y_perm, None, ws)
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    moe.moe_combine(s, y_perm, slot_pos, layer.topk_w, y)
    torch.cuda.synchronize()
    y_un = y.cpu().numpy()
    # same routing, same bf16 hidden rows: the two combines differ only in
    # fp32 summation order
    assert rel_err(y_un, out["y"]) < 1e-5
    out2 = dict(out)
    out2["y"] = y_un
    check_forward(wl, out2)


@pytest.mark.parametrize("form", ["fused", "grouped"])
def test_combine_forms(moe, form):
    """Both combine forms of moe_forward against the oracle: fp32 atomic adds
    in the down projection (the default at decode sizes), and a grouped
    output summed by the combine pass, on a shape with k = 4, a shared expert
    and a capacity limit."""
    cfg = custom_config(400, 256, 16, 4, 256, shared=True, cf=1.25, seed=41)
    wl = Workload(cfg)
    out, _, _ = gpu_forward(wl, combine=form)
    rep = check_forward(wl, out)
    print(f"[combine {form}] err={rep['err']:.3e}", flush=True)


def test_grouped_combine_is_deterministic(moe):
    """The grouped-output combine sums in slot order: two runs are bit-equal
    even with k = 8 and a shared expert."""
    cfg = custom_config(300, 256, 32, 8, 128, shared=True, seed=43)
    wl = Workload(cfg)
    out1, layer, dev = gpu_forward(wl, combine="grouped")
    layer(dev["x"])
    torch.cuda.synchronize()
    assert np.array_equal(layer.y.cpu().numpy(), out1["y"])


def test_T0_is_a_noop(moe):
    s = moe.make_shape(0, 256, 8, 2, 128)
    ws = moe.workspace(s)
    z = torch.zeros(1, device="cuda")
    counts = torch.full((8,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.full((9,), -1, dtype=torch.int32, device="cuda")
    wts = moe.make_weights(W1=z, W3=z, W2=z)
    moe.moe_forward(s, None, None, None, wts, None, None, None, counts, offsets, ws)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 8 and offsets.cpu().tolist() == [0] * 9


def test_determinism_k2(moe):
    """The fused (atomic) combine with k = 2 and an unsplit down projection
    (d_ff = 256: one K piece per tile): every y element receives two fp32
    adds onto zero, which commute, so two runs are bit-identical."""
    cfg = custom_config(900, 512, 8, 2, 256, seed=77)
    wl = Workload(cfg)
    out1, layer, dev = gpu_forward(wl, combine="fused")
    layer(dev["x"])
    torch.cuda.synchronize()
    assert np.array_equal(layer.topk_idx.cpu().numpy(), out1["idx"])
    assert np.array_equal(layer.topk_w.cpu().numpy(), out1["w"])
    assert np.array_equal(layer.y.cpu().numpy(), out1["y"])


def test_decode_sized_reproducibility(moe):
    """A decode-sized batch with a long down-projection K (d_ff = 4096): the
    fused combine splits each down tile over K, so a y element receives
    k * pieces fp32 atomic adds in an order that can change between runs
    (two runs agree within the tolerance, not necessarily bit for bit); the
    grouped combine sums the pieces and the rows in a fixed order, so two
    runs are bit-identical."""
    cfg = custom_config(64, 1024, 8, 2, 4096, seed=78)
    wl = Workload(cfg)
    out_g, layer_g, dev = gpu_forward(wl, combine="grouped")
    layer_g(dev["x"])
    torch.cuda.synchronize()
    assert np.array_equal(layer_g.y.cpu().numpy(), out_g["y"])
    out_f, layer_f, _ = gpu_forward(wl, combine="fused", dev=dev)
    layer_f(dev["x"])
    torch.cuda.synchronize()
    assert rel_err(layer_f.y.cpu().numpy(), out_f["y"]) < 1e-5
    assert rel_err(out_f["y"], out_g["y"]) < 1e-5
    check_forward(wl, out_f)


def _full_size(wl, **kw):
    """moe_forward at full size, then the oracle on every token, fed from the
    host copies of the uploaded weights."""
    host = {}
    out, layer, dev = gpu_forward(wl, keep_host=host, **kw)
    stream = ExpertStream(lambda e: host[e], wl.cfg.E, expert_bytes_f64(wl.cfg))
    return out, layer, dev, stream


@pytest.mark.parametrize("name", ["mixtral", "decode", "capacity_skew", "fine_grained",
                                  "fine_grained_fp8", "fine_grained_int8", "fine_grained_int4",
                                  "decode_int4", "decode_fp8", "decode_int8"])
def test_workload_full_size(moe, name):
    """Every token of the named workload against the oracle.  The fine-grained
    layer's 256 experts each hold about 128 rows, so every expert segment and
    every 256-row tile of the shared expert is compared."""
    print(f"[workload] {name}", flush=True)
    wl = Workload(get_config(name))
    out, _, _, stream = _full_size(wl)
    try:
        rep = check_forward(wl, out, experts=stream)
    finally:
        stream.close()
    print(f"  err={rep['err']:.3e} (nonzero rows {rep['nonzero_rows']}: "
          f"{rep['err_nonzero_rows']:.3e}) tokens={rep['tokens']} flipped={rep['flipped']} "
          f"kept={rep['kept']}", flush=True)
    assert rep["tokens"] == wl.cfg.T


class _Int4WithMinus8(Workload):
    """The synthetic int4 weights with about 6% of the codes set to -8 (nibble
    0), which the format accepts but the quantiser never writes."""

    def _poke(self, w, seed):
        rng = np.random.default_rng(seed)
        for n in ("W1", "W3", "W2"):
            a = np.ascontiguousarray(w[n]).view(np.uint8).copy()
            lo = rng.random(a.shape) < 0.06
            hi = rng.random(a.shape) < 0.06
            a[lo] &= 0xF0
            a[hi] &= 0x0F
            w[n] = a.view(INT4X2)
        return w

    def expert(self, e):
        return self._poke(super().expert(e), 1000 + e)

    def shared(self):
        w = super().shared()
        return None if w is None else self._poke(w, 999)


@pytest.mark.parametrize("T,d,E,k,d_ff,shared", [(700, 512, 8, 2, 384, True),
                                                  (64, 512, 8, 2, 1408, False),
                                                  (300, 4096, 4, 2, 256, False)])
def test_int4_code_minus8(moe, T, d, E, k, d_ff, shared):
    cfg = custom_config(T, d, E, k, d_ff, w="int4", shared=shared, seed=T + 17)
    wl = _Int4WithMinus8(cfg)
    w0 = np.ascontiguousarray(wl.expert(0)["W1"]).view(np.uint8)
    assert ((w0 & 0x0F) == 0).any() and ((w0 >> 4) == 0).any()
    out, _, _ = gpu_forward(wl)
    rep = check_forward(wl, out)
    print(f"[int4 -8] T={T} d={d} err={rep['err']:.3e}", flush=True)


@pytest.mark.parametrize("T,d,E,k,d_ff,cf,shared,w,G,M", [
    (600, 256, 16, 4, 256, None, False, "bf16", 4, 2),
    (500, 512, 32, 6, 128, 1.25, True, "bf16", 8, 3),
    (300, 256, 64, 8, 128, None, True, "fp8_e4m3", 8, 4)])
def test_forward_group_limited(moe, T, d, E, k, d_ff, cf, shared, w, G, M):
    """Group-limited routing end to end; routing decided on the GPU's fp32
    logits on both sides (the logits checked against the oracle's)."""
    print(f"[forward groups] T={T} E={E} k={k} G={G} M={M} cf={cf} shared={shared} w={w}",
          flush=True)
    cfg = custom_config(T, d, E, k, d_ff, w=w, cf=cf, shared=shared, seed=T + 5 * E)
    wl = Workload(cfg)
    out, layer, dev = gpu_forward(wl, groups=G, topk_groups=M)
    gl = gpu_logits(layer, dev)
    rep = check_forward(wl, out, decide_on=gl, groups=G, topk_groups=M)
    idx = out["idx"]
    assert all(len({int(e) // (E // G) for e in row}) <= M for row in idx)
    print(f"  err={rep['err']:.3e} kept={rep['kept']}", flush=True)


def test_fine_grained_group_limited_full_size(moe):
    """The 256-expert layer (k = 8 + a shared expert) with 8 groups of 32
    experts and at most 4 groups per token, at full size."""
    print("[workload] fine_grained, 8 groups, top-4 groups", flush=True)
    wl = Workload(get_config("fine_grained"))
    out, layer, dev, stream = _full_size(wl, groups=8, topk_groups=4)
    gl = gpu_logits(layer, dev)
    try:
        rep = check_forward(wl, out, decide_on=gl, groups=8, topk_groups=4, experts=stream)
    finally:
        stream.close()
    assert rep["tokens"] == wl.cfg.T
    print(f"  err={rep['err']:.3e} kept={rep['kept']}", flush=True)

