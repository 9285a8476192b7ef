"""Helpers that run the HIP path through the C ABI and compare it with the oracle.

Used by the GPU tests, the smoke check and the benchmark's parity line.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle
from moe_synth import Workload

MARGIN_EXCLUDE = 1e-5            # tokens with a smaller top-k margin may flip
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8_e4m3": 6e-2, "int8": 2e-2, "int4": 2e-2}
LOGIT_TOL = 1e-4                 # fp32 router logits against the float64 oracle


class ExpertStream:
    """expert(e) for the oracle's loops over experts: each routed expert's
    matrices decoded to float64 by the oracle's own weight decoding, prepared
    ahead on a thread pool in increasing expert order (the order in which the
    oracle visits experts), so its sequential loop does not wait for input
    generation.  source(e) gives the expert's weights as stored (codes and
    scales for the quantised formats).  The decoded arrays are what the
    oracle would compute from source(e) itself."""

    def __init__(self, source, E: int, per_expert_bytes: int, workers=None,
                 budget_bytes=8 << 30):
        self.source = source
        self.E = E
        self.ahead = int(max(2, min(32, budget_bytes // max(per_expert_bytes, 1))))
        n = workers or max(1, min(16, len(os.sched_getaffinity(0))) - 1)
        self.pool = cf.ThreadPoolExecutor(max_workers=n)
        self.futs = {}
        self.next = 0

    def _decode(self, e):
        w = self.source(e)
        names = [n for n in ("W1", "W3", "W2", "W", "b") if n in w]
        out = {n: oracle.moe_oracle._weight(w, n) for n in names if n != "b"}
        if "b" in w:
            out["b"] = w["b"]
        return out

    def __call__(self, e: int) -> dict:
        e = int(e)
        for old in [k for k in self.futs if k < e]:
            self.futs.pop(old).cancel()
        self.next = max(self.next, e)
        while self.next < min(self.E, e + self.ahead):
            self.futs[self.next] = self.pool.submit(self._decode, self.next)
            self.next += 1
        f = self.futs.pop(e, None)
        return f.result() if f is not None else self._decode(e)

    def close(self):
        for f in self.futs.values():
            f.cancel()
        self.pool.shutdown(wait=True)


def expert_bytes_f64(cfg) -> int:
    if cfg.kind == "linear_bias":
        return cfg.d * cfg.d * 8
    return 3 * cfg.d * cfg.d_ff * 8


def tolerance(cfg) -> float:
    return TOL["f32"] if cfg.kind == "linear_bias" else TOL[cfg.w]


def oracle_capacity(cfg) -> int:
    return oracle.capacity(cfg.T, cfg.E, cfg.k, cfg.cf)


def gpu_forward(wl: Workload, dev=None, overflow="drop", rounds=0, groups=0, topk_groups=0,
                combine="auto", keep_host=None):
    """Run moe_forward once on the workload; returns (numpy outputs, layer, dev).
    combine: "auto", "grouped" or "fused" (moe_shape.combine)."""
    import torch

    import mixture_experts_layer_bincount_amd as moe
    from moe_synth.device import upload
    c = wl.cfg
    if dev is None:
        dev = upload(wl, keep_host=keep_host)
    cap = moe.moe_capacity(c.T, c.E, c.k, c.cf) if c.cf else -1
    layer = moe.MoELayer(c.T, c.d, c.E, c.k, c.d_ff, W_g=dev["W_g"], b_g=dev["b_g"],
                         weights=dev["weights"], capacity=cap, kind=c.kind, w_dtype=c.w,
                         has_shared=c.shared, overflow=overflow, reroute_rounds=rounds,
                         n_groups=groups, topk_groups=topk_groups, combine=combine,
                         hidden_split=c.hidden_split)
    layer(dev["x"])
    torch.cuda.synchronize()
    out = dict(y=layer.y.cpu().numpy(), idx=layer.topk_idx.cpu().numpy(),
               w=layer.topk_w.cpu().numpy(), counts=layer.counts.cpu().numpy(),
               offsets=layer.offsets.cpu().numpy())
    return out, layer, dev


def gpu_logits(layer, dev) -> np.ndarray:
    """The router logits moe_forward decides on: moe_route on the same shape
    runs the same router kernels in the same configuration, so its fp32
    logits are those moe_forward's selection (and re-routing) used."""
    import torch

    import mixture_experts_layer_bincount_amd as moe
    s = layer.shape
    logits = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((s.T, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((s.T, s.top_k), dtype=torch.float32, device="cuda")
    W_g = layer.W_g_packed if layer.W_g_packed is not None else dev["W_g"]
    moe.moe_route(s, dev["x"], W_g, dev["b_g"], logits, idx, w, moe.workspace(s))
    torch.cuda.synchronize()
    return logits.cpu().numpy()


def check_routing(logits, k, gpu_idx, gpu_w, w_tol=1e-5):
    """Indices equal except on tokens whose top-k margin is below 1e-5; weights
    of the equal tokens within w_tol.  Returns the mask of flipped tokens."""
    o_idx, o_w = oracle.route(logits, k)
    margin = oracle.topk_margin(logits, k)
    flip = (gpu_idx != o_idx).any(axis=1)
    bad = flip & (margin >= MARGIN_EXCLUDE)
    assert not bad.any(), (f"{bad.sum()} tokens with margin >= {MARGIN_EXCLUDE} routed "
                           f"differently, first {np.nonzero(bad)[0][:5]}")
    same = ~flip
    if same.any():
        err = np.abs(gpu_w[same] - o_w[same]).max()
        assert err <= w_tol, f"routing weights differ by {err}"
    return flip


def rel_err(y, y_ref) -> float:
    rms = float(np.sqrt(np.mean(np.square(y_ref))))
    return float(np.abs(y - y_ref).max() / max(rms, 1e-30))


def check_forward(wl: Workload, gpu: dict, tokens=None, tol=None, overflow="drop", rounds=0,
                  decide_on=None, groups=0, topk_groups=0, experts=None) -> dict:
    """Compare one moe_forward result with the oracle (on all tokens, or on
    the sampled `tokens`).  Returns a report dict.

    decide_on: the GPU's fp32 logits (gpu_logits()).  When given, the
    oracle's routing decisions (top-k, and the ranking that re-routing
    follows past the top-k) are taken on those same fp32 values, after the
    logits themselves are checked against the oracle's float64 logits.

    experts: the oracle's expert(e) (default: the workload's generator);
    an ExpertStream over the same weights serves large workloads.

    The report also holds err_nonzero_rows: the same ratio over the rows
    where the oracle's y is not zero (tokens whose assignments all drop have
    y = 0 on both sides and dilute RMS(y) otherwise)."""
    c = wl.cfg
    C = oracle_capacity(c)
    x = wl.x()
    W_g = wl.W_g()
    b_g = wl.b_g()
    logits = oracle.router_logits(x, W_g, b_g)
    if decide_on is None:
        assert groups <= 1, "group-limited routing is checked on the GPU's logits"
        flip = check_routing(logits, c.k, gpu["idx"], gpu["w"])
        override = gpu["idx"] if flip.any() else None
    else:
        lerr = rel_err(decide_on.astype(np.float64), logits)
        assert lerr <= LOGIT_TOL, f"router logits: max-abs-err/RMS = {lerr:.3e}"
        o_idx, o_w = oracle.route(decide_on, c.k, groups, topk_groups)
        assert np.array_equal(gpu["idx"], o_idx), "top-k differs on the same fp32 logits"
        assert np.abs(gpu["w"] - o_w).max() <= 1e-5, "routing weights differ"
        logits = decide_on.astype(np.float64)
        flip = np.zeros(c.T, dtype=bool)
        override = None
    shared = wl.shared if c.shared else None
    experts = experts or wl.expert
    pol = dict(overflow=overflow, rounds=rounds, groups=groups, topk_groups=topk_groups)
    if tokens is None:
        r = oracle.forward(x, W_g, b_g, c.k, c.E, experts, kind=c.kind, C=C,
                           shared=shared, idx_override=override, logits=logits, **pol)
        y_ref = r["y"]
        y = gpu["y"]
    else:
        tokens = np.asarray(tokens)
        y_ref, r = oracle.forward_tokens(tokens, x, W_g, b_g, c.k, c.E, experts, kind=c.kind,
                                         C=C, shared=shared, idx_override=override,
                                         logits=logits, **pol)
        y = gpu["y"][tokens]
    # load accounting is bit-exact given the same selection
    assert np.array_equal(gpu["counts"], r["counts"]), "counts differ"
    assert np.array_equal(gpu["offsets"], r["offsets"]), "offsets differ"
    err = rel_err(y, y_ref)
    nz = np.any(y_ref != 0.0, axis=1)
    err_nz = rel_err(y[nz], y_ref[nz]) if nz.any() else 0.0
    tol = tolerance(c) if tol is None else tol
    assert err <= tol, f"max-abs-err/RMS = {err:.3e} > {tol}"
    return dict(err=err, err_nonzero_rows=err_nz, nonzero_rows=int(nz.sum()),
                tokens=int(y_ref.shape[0]), flipped=int(flip.sum()), tol=tol,
                kept=int(r["offsets"][-1]), counts=r["counts"], C=C)
