#!/usr/bin/env python3
"""Benchmark of the MoE FFN layer forward pass on one MI355X.

Headline workload: the Mixtral-shaped layer (T=4096 tokens, d=4096, E=8
experts, top-2, SwiGLU experts with d_ff=14336, bf16 activations and
weights, fp32 router, no capacity limit), synthetic seeded inputs resident
in HBM before the timed region.  One step = one full moe_forward (router,
top-k, dispatch, grouped gate/up GEMM + SwiGLU, grouped down GEMM, combine).
The timed region runs without any instrumentation; a second pass of the same
steps records HIP events around each stage on the launch stream, which give
the dominant kernel's duration for the roofline line.

Prints one JSON line.  Also reported:
  parity        the timed run's y against the CPU oracle on every token
  decode_t64    the decode-shaped layer (the same weights, T=64), HBM GB/s
                over the touched expert weights
  workloads     one record per other workload (the tutorial-sized layer, the
                capacity-limited skewed layer with its load report, the
                fine-grained layer in bf16 and with fp8 weights): step time
                and the fraction of its binding roofline floor
  cpu_baseline  the CPU oracle timed on a bounded sample of the headline
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "MoE-layer tokens/s (Mixtral shape, T=4096) + % MFMA peak; decode T=64 % HBM BW"
SUB_WORKLOADS = ("tiny", "capacity_skew", "fine_grained", "fine_grained_fp8")
# parity bounds on max-abs error / RMS(y): fp32 Linear+bias layer, bf16 (and
# int8 / int4) weights, fp8 weights
TOL = {"f32": 1e-4, "bf16": 2e-2, "int8": 2e-2, "int4": 2e-2, "fp8_e4m3": 6e-2}


def tolerance(cfg) -> float:
    return TOL["f32"] if cfg.kind == "linear_bias" else TOL[cfg.w]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def _traffic_from_profile(kernel_src: str, key: str, workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary of the Mixtral-shaped workload, or None for another
    workload or when the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "gate_up_swiglu_mixtral_counters.json")
    if workload != "mixtral" or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(kernel_src, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()
    if rec.get("kernel_source_sha256") != h:
        return None
    return rec.get(key)


# ---------------------------------------------------------------- workloads
class Loaded:
    """One workload's inputs on the device and its layer (argument plumbing)."""

    def __init__(self, name, overflow="drop", rounds=0, groups=0, topk_groups=0,
                 host_experts=None, dev_w=None, x=None, W_g=None, b_g=None):
        import numpy as np

        import mixture_experts_layer_bincount_amd as moe
        from moe_synth import Workload, get_config
        from moe_synth.device import to_device

        self.cfg = cfg = get_config(name)
        self.wl = wl = Workload(cfg)
        self.host_experts = host_experts
        if dev_w is None:
            log(f"generating {cfg.name} inputs")
            keep = {} if host_experts is None else host_experts
            dev_w = {}
            if cfg.kind == "linear_bias":
                ws = [wl.expert(e) for e in range(cfg.E)]
                for n in ws[0]:
                    dev_w[n] = to_device(np.stack([w[n] for w in ws]), "cuda")
                keep.update(dict(enumerate(ws)))
            else:
                first = wl.expert(0)
                for n, a in first.items():
                    t = to_device(a[:1], "cpu")
                    dev_w[n] = torch_empty((cfg.E,) + a.shape, t.dtype)

                def put(e, w):
                    for n, a in w.items():
                        dev_w[n][e].copy_(to_device(a, "cpu"))
                    if host_experts is not None:
                        keep[e] = w

                wl.experts_parallel(range(cfg.E), put)
                sh = wl.shared()
                if sh is not None:
                    for n, a in sh.items():
                        dev_w[n + "s"] = to_device(a, "cuda")
        self.dev_w = dev_w
        self.x = x if x is not None else to_device(wl.x(), "cuda")
        self.W_g = W_g if W_g is not None else to_device(wl.W_g(), "cuda")
        if b_g is None and wl.b_g() is not None:
            b_g = to_device(wl.b_g(), "cuda")
        self.b_g = b_g
        self.cap = moe.moe_capacity(cfg.T, cfg.E, cfg.k, cfg.cf) if cfg.cf else -1
        self.layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, W_g=self.W_g,
                                  b_g=self.b_g, weights=dev_w, capacity=self.cap, kind=cfg.kind,
                                  w_dtype=cfg.w, has_shared=cfg.shared, overflow=overflow,
                                  reroute_rounds=rounds, n_groups=groups,
                                  topk_groups=topk_groups, hidden_split=cfg.hidden_split)

    def step(self):
        return self.layer(self.x)


def torch_empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def time_steps(fn, steps: int) -> float:
    """ms per step over `steps` calls, bracketed by device synchronisations."""
    import torch
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def ffn_flops(cfg, kept: int) -> float:
    """Expert FFN FLOPs of one step: 2*3*d*d_ff per kept assignment, plus the
    shared expert over every token (SwiGLU); 2*d*d per assignment for the
    Linear+bias experts."""
    if cfg.kind == "linear_bias":
        return 2.0 * kept * cfg.d * cfg.d
    f = 2.0 * 3 * cfg.d * cfg.d_ff * kept
    if cfg.shared:
        f += 2.0 * 3 * cfg.d * cfg.d_ff * cfg.T
    return f


def weight_bytes(cfg, n_experts: int) -> int:
    """Bytes of n_experts experts' weights in the workload's format (codes and
    their fp32 scales for the quantised formats)."""
    wbits = {"bf16": 16, "fp8_e4m3": 8, "int8": 8, "int4": 4, "f32": 32}[cfg.w]
    if cfg.kind == "linear_bias":
        return n_experts * (cfg.d * cfg.d + cfg.d) * 4
    per = 3 * cfg.d * cfg.d_ff * wbits // 8
    if wbits < 16:
        per += 4 * (2 * cfg.d_ff + cfg.d) // 128
    return n_experts * per


def gemm_kernel(cfg, cap: int, stage: str = "gate_up") -> str:
    """The expert GEMM kernel the library launches for one stage ("gate_up"
    or "down") of this workload.  The choice follows the average rows per
    expert, P_max / E with P_max = min(T k, E C): up to 32 rows the four-wave
    kernel with decode-sized activation tiles; otherwise the eight-wave
    ping-pong kernel for bf16 weights and for 8-bit weights from 256 rows
    up, its 128 x 512 tiles for the down projection of 8-bit weights with
    fewer rows; the four-wave kernel with 256-row tiles for int4 and for the
    gate/up projection of 8-bit weights with fewer rows."""
    if cfg.kind != "swiglu":
        return "linear_bias_kernel"
    A = cfg.T * cfg.k
    rows = (A if cap < 0 else min(A, cfg.E * cap)) // cfg.E
    if rows <= 32:
        return "grouped_gemm_dma_kernel (decode-sized tiles)"
    if cfg.w == "bf16" or (cfg.w in ("fp8_e4m3", "int8") and rows >= 256):
        return "grouped_gemm_pp_kernel"
    if cfg.w in ("fp8_e4m3", "int8") and stage == "down":
        return "grouped_gemm_pp_kernel (128 x 512 tiles)"
    return "grouped_gemm_dma_kernel"


def gate_up_bytes(cfg, kept_rows) -> int:
    """Algorithmic bytes of the gate/up launch: W1 and W3 of the experts it
    touches (codes and scales in the workload's format, the shared expert
    included), the gathered x rows read once, H written once."""
    wbits = {"bf16": 16, "fp8_e4m3": 8, "int8": 8, "int4": 4}[cfg.w]
    n = sum(1 for v in kept_rows if v > 0) + (1 if cfg.shared else 0)
    w = n * 2 * cfg.d * cfg.d_ff * wbits // 8
    if wbits < 16:
        w += n * 2 * (cfg.d_ff // 128) * 4
    rows = int(sum(kept_rows)) + (cfg.T if cfg.shared else 0)
    return w + rows * cfg.d * 2 + rows * cfg.d_ff * 2 * (2 if cfg.hidden_split else 1)


def roofline_floor(cfg, kept_rows, kept: int) -> dict:
    """The binding floor of one step: max(MFMA time of the expert FLOPs at
    2.5 PFLOP/s, HBM time of the touched weights + x read once + y written
    once at 8 TB/s)."""
    touched = sum(1 for v in kept_rows if v > 0) + (1 if cfg.shared else 0)
    wb = weight_bytes(cfg, touched)
    xb = cfg.T * cfg.d * (4 if cfg.act == "f32" else 2)
    yb = cfg.T * cfg.d * 4
    hbm_bytes = wb + xb + yb
    fl = ffn_flops(cfg, kept)
    t_mfma = fl / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    t_hbm = hbm_bytes / (PEAK_HBM_GBS * 1e9) * 1e3
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    return {"bound": bound, "floor_ms": max(t_mfma, t_hbm), "mfma_floor_ms": t_mfma,
            "hbm_floor_ms": t_hbm, "ffn_flops": fl, "hbm_bytes": hbm_bytes,
            "touched_experts": touched}


def load_stats(moe, counts, kept_rows) -> dict:
    """Tutorial §4.2 / §4.3: the imbalance max/(min + 1e-6) and the LPT packing
    of the loads onto 8 devices, by the library's host functions, on the raw
    counts and on the kept (capacity-limited) rows."""
    stats = {}
    for name, load in (("counts", counts), ("kept", kept_rows)):
        _, bins = moe.moe_lpt_pack(load, 8)
        stats[name] = {"imbalance": moe.moe_load_imbalance(load),
                       "max": int(max(load)), "min": int(min(load)),
                       "max_over_mean": max(load) / (sum(load) / len(load)),
                       "empty_experts": int(sum(1 for v in load if v == 0)),
                       "lpt_8_bins": bins,
                       "lpt_8_max_over_mean": max(bins) / (sum(bins) / len(bins))}
    return stats


# ---------------------------------------------------------------- CPU baseline leg
# The only code here that runs the CPU oracle: it times the oracle and keeps
# its outputs, against which the GPU results of the same inputs are compared.
def oracle_reference(L: Loaded, n_tokens=None):
    """The oracle's y on the first n_tokens tokens (all when None) of L's
    workload, and the seconds it took (float64 NumPy on the host cores)."""
    import oracle
    c = L.cfg
    n = c.T if n_tokens is None else min(n_tokens, c.T)
    experts = (lambda e: L.host_experts[e]) if L.host_experts else L.wl.expert
    x = L.wl.x()[:n]
    t0 = time.perf_counter()
    r = oracle.forward(x, L.wl.W_g(), L.wl.b_g(), c.k, c.E, experts, kind=c.kind,
                       C=oracle.capacity(n, c.E, c.k, c.cf),
                       shared=L.wl.shared if c.shared else None)
    return r["y"], time.perf_counter() - t0


def parity_report(cfg, y, y_ref) -> dict:
    """max-abs error / RMS of y against the oracle's y_ref, plus the same
    ratio over the rows the oracle's y is not zero on (the kept rows; a token
    whose assignments all drop has y = 0 on both sides)."""
    import numpy as np
    err = float(np.abs(y - y_ref).max() / np.sqrt(np.mean(np.square(y_ref))))
    out = {"err": err, "tol": tolerance(cfg), "tokens": int(y_ref.shape[0]),
           "ok": bool(err <= tolerance(cfg))}
    nz = np.any(y_ref != 0.0, axis=1)
    if nz.sum() < nz.size:
        yk, yr = y[nz], y_ref[nz]
        out["err_nonzero_rows"] = float(np.abs(yk - yr).max() / np.sqrt(np.mean(np.square(yr))))
        out["nonzero_rows"] = int(nz.sum())
    return out


def sub_record(name: str, steps: int, warmup: int, parity: bool) -> dict:
    """Step time of one workload against its binding floor."""
    import numpy as np

    import mixture_experts_layer_bincount_amd as moe
    L = Loaded(name, host_experts={} if parity else None)
    for _ in range(warmup):
        L.step()
    ms = time_steps(L.step, steps)
    c = L.cfg
    kept_rows = np.diff(L.layer.offsets.cpu().numpy()).tolist()
    kept = int(sum(kept_rows))
    counts = L.layer.counts.cpu().tolist()
    floor = roofline_floor(c, kept_rows, kept)
    rec = {"config": {"T": c.T, "d": c.d, "E": c.E, "top_k": c.k, "d_ff": c.d_ff,
                      "expert": c.kind, "weights": c.w, "shared": c.shared,
                      "capacity": L.cap, "hidden_split": c.hidden_split},
           "steps": steps, "ms_per_step": ms, "tokens_per_s": c.T / (ms * 1e-3),
           "kept_assignments": kept,
           "gemm_kernels": {"gate_up": gemm_kernel(c, L.cap), "down": gemm_kernel(c, L.cap, "down")},
           **floor,
           "frac": floor["floor_ms"] / ms,
           "tflops": floor["ffn_flops"] / (ms * 1e-3) / 1e12,
           "hbm_gbs_over_step": floor["hbm_bytes"] / (ms * 1e-3) / 1e9}
    if c.cf or c.router_bias:
        rec["load_stats"] = load_stats(moe, counts, kept_rows)
    if parity:
        y = L.layer.y.cpu().numpy()
        y_ref, secs = oracle_reference(L)
        rec["parity"] = parity_report(c, y, y_ref)
        rec["parity"]["oracle_s"] = secs
    log(f"{name}: {ms:.3f} ms/step, {rec['frac']:.3f} of its {floor['bound']} floor")
    del L
    return rec


def cpu_baseline(L: Loaded, n_tokens: int, repeats: int) -> tuple:
    """The oracle as it stands, on the first n_tokens tokens of the workload
    (routing, dispatch, masked per-expert loop, combine; float64), run
    `repeats` times.  Returns (record, the last run's y, tokens)."""
    c = L.cfg
    n_tokens = min(n_tokens, c.T)
    dt = 0.0
    for _ in range(repeats):
        y, secs = oracle_reference(L, n_tokens)
        dt += secs
    rec = {"value": n_tokens * repeats / dt, "unit": "tokens/s", "cores": _blas_threads(),
           "kind": "oracle",
           "sample": f"first {n_tokens} of the {c.T} tokens of the {c.name} workload, whole "
                     f"layer (router, top-k, bincount, dispatch, masked per-expert loop, "
                     f"combine) in float64 NumPy, {repeats} runs; {dt:.1f} s on {_cpu_model()}"}
    return rec, y, n_tokens


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--sub-steps", type=int, default=20)
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-sub", action="store_true", help="skip the other workloads' records")
    ap.add_argument("--overflow", default="drop", choices=("drop", "reroute", "shared"),
                    help="fate of assignments past the capacity")
    ap.add_argument("--rounds", type=int, default=1, help="re-routing rounds (--overflow reroute)")
    ap.add_argument("--groups", type=int, default=0,
                    help="group-limited routing: expert groups (0 = off)")
    ap.add_argument("--topk-groups", type=int, default=0, help="groups a token may use")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer runs on one GPU's share of tokens, with no collectives)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mixture_experts_layer_bincount_amd as moe
    from moe_synth import get_config

    torch.cuda.set_device(0)
    rounds = args.rounds if args.overflow == "reroute" else 0
    H = Loaded(args.workload, overflow=args.overflow, rounds=rounds, groups=args.groups,
               topk_groups=args.topk_groups, host_experts={})
    cfg = H.cfg
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        H.step()
    torch.cuda.synchronize()

    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- timed region: K steps, nothing else on the stream
    ms_per_step = time_steps(H.step, args.steps)
    log(f"{args.steps} steps, {ms_per_step:.3f} ms/step")

    # ---- roofline pass: the same K steps with HIP events recorded on the
    # launch stream around each stage (the dominant kernel's duration)
    moe.moe_timing_enable(True)
    moe.moe_timing_collect()
    ms_instrumented = time_steps(H.step, args.steps)
    stage_ms, calls = moe.moe_timing_collect()
    moe.moe_timing_enable(False)

    kept_rows = np.diff(H.layer.offsets.cpu().numpy()).tolist()
    kept = int(sum(kept_rows))
    counts = H.layer.counts.cpu().tolist()
    y_gpu = H.layer.y.cpu().numpy()
    rows_gu = kept + (cfg.T if cfg.shared else 0)  # the shared expert runs over every token
    flops_gate_up = 2.0 * rows_gu * cfg.d * 2 * cfg.d_ff
    flops_down = 2.0 * rows_gu * cfg.d_ff * cfg.d
    flops_ffn = ffn_flops(cfg, kept)
    gu_ms = stage_ms["gate_up_swiglu"] / max(calls, 1)
    dn_ms = stage_ms["down_combine"] / max(calls, 1)
    achieved = flops_gate_up / (gu_ms * 1e-3) / 1e12
    gemm_src = os.path.join(ROOT, "mixture_experts_layer_bincount_amd", "csrc", "expert_gemm.hip")
    traffic = _traffic_from_profile(gemm_src, "hbm_bytes_per_launch", cfg.name)
    stages = {k: round(v / max(calls, 1), 4) for k, v in stage_ms.items()}

    result = {
        "metric": METRIC,
        "value": cfg.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} MoE FFN layer", "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "top_k": cfg.k, "d_ff": cfg.d_ff, "expert": "SwiGLU", "router": "fp32",
                   "capacity": H.cap, "overflow": args.overflow, "reroute_rounds": rounds,
                   "groups": args.groups, "topk_groups": args.topk_groups,
                   "global_batch": cfg.T, "parallelism": "none (1 GPU)"},
        "layer_mfma_frac": flops_ffn / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "layer_tflops": flops_ffn / (ms_per_step * 1e-3) / 1e12,
        "stage_ms": stages,
        "ms_per_step_stage_timed": ms_instrumented,
        "counts": counts,
        "roofline": {"kernel": f"grouped gate/up GEMM + SwiGLU ({gemm_kernel(cfg, H.cap)}<GATEUP>)",
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "algorithmic_per_launch": f"{flops_gate_up:.4e} FLOP = 2*{rows_gu} rows*"
                                               f"{cfg.d}*2*{cfg.d_ff}",
                     "avg_launch_ms": gu_ms,
                     "timing": f"HIP events on the launch stream around the launch, "
                               f"{calls} steps after the timed region",
                     "down_combine": {"avg_launch_ms": dn_ms,
                                      "tflops": flops_down / (dn_ms * 1e-3) / 1e12}},
        "load_stats": load_stats(moe, counts, kept_rows),
    }
    # a workload whose binding floor is the HBM (decode-sized batches, the
    # 256-expert layer): the gate/up launch's algorithmic bytes per second
    # against 8 TB/s
    floor = roofline_floor(cfg, kept_rows, kept) if cfg.kind == "swiglu" else None
    if floor and floor["bound"] == "hbm":
        gb = gate_up_bytes(cfg, kept_rows)
        r = result["roofline"]
        r.update({"bound": "hbm", "achieved": gb / (gu_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                  "unit": "GB/s", "frac": gb / (gu_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "algorithmic_per_launch": f"{gb:.4e} B = W1 + W3 of the touched experts "
                                            f"+ {rows_gu} gathered x rows + H",
                  "tflops": achieved})

    # ---- weight stream: the bytes of the experts this step touched (codes
    # and scales in the workload's weight format, the shared expert included)
    if cfg.kind == "swiglu":
        n_exp = sum(1 for v in kept_rows if v > 0) + (1 if cfg.shared else 0)
        wb = weight_bytes(cfg, n_exp)
        result["weight_stream"] = {
            "experts": n_exp, "bytes": wb,
            "gbs_over_step": wb / (ms_per_step * 1e-3) / 1e9,
            "hbm_frac_over_step": wb / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "gbs_over_ffn_stages": wb / ((gu_ms + dn_ms) * 1e-3) / 1e9}

    # ---- the one-time router packing the layer did at construction (outside
    # moe_forward, so outside the timed steps), timed on its own
    if H.layer.W_g_packed is not None:
        pk = lambda: moe.moe_pack_router(H.layer.shape, H.W_g, H.layer.W_g_packed)  # noqa: E731
        pk()
        result["router_pack"] = {"bytes": int(H.layer.W_g_packed.numel()),
                                 "us_once": time_steps(pk, 10) * 1e3,
                                 "note": "moe_pack_router, once per layer, not in the timed steps"}

    # ---- online EPLB on the device: replicas + placement onto 8 devices from
    # this step's counts (still on the device), E/8 extra replicas
    D, extra = 8, max(1, cfg.E // 8)
    reps = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    sdev = torch.empty(cfg.E + extra, dtype=torch.int32, device="cuda")
    sload = torch.empty(cfg.E + extra, dtype=torch.int32, device="cuda")
    dload = torch.empty(D, dtype=torch.int64, device="cuda")
    plan = lambda: moe.moe_eplb_plan(H.layer.counts, D, extra, reps, sdev, sload, dload)  # noqa: E731
    for _ in range(3):
        plan()
    us_plan = time_steps(plan, 20) * 1e3
    dl = dload.cpu().numpy()
    result["eplb_plan"] = {"devices": D, "extra_replicas": extra, "us_per_plan": us_plan,
                           "device_load_max_over_mean": float(dl.max() / dl.mean()),
                           "without_replicas_max_over_mean":
                               result["load_stats"]["counts"]["lpt_8_max_over_mean"]}

    # ---- decode-shaped layer: the same weights, the first 64 tokens
    if not args.no_decode and cfg.name == "mixtral":
        dcfg = get_config("decode")
        xd = H.x[: dcfg.T].contiguous()
        D_ = moe.MoELayer(dcfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, W_g=H.W_g, b_g=H.b_g,
                          weights=H.dev_w, kind=cfg.kind, w_dtype=cfg.w)
        step = lambda: D_(xd)  # noqa: E731
        for _ in range(5):
            step()
        dms = time_steps(step, args.decode_steps)
        # the same decode step replayed from a captured HIP graph (no
        # per-kernel launch cost on the host side)
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            step()
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        dms_graph = time_steps(graph.replay, args.decode_steps)
        dcounts = D_.counts.cpu().numpy()
        touched = int((dcounts > 0).sum())
        wbytes = weight_bytes(cfg, touched)
        yd = D_.y.cpu().numpy()
        # decode parity: the oracle on the same 64 tokens (the decode layer's
        # x is the first 64 rows of the headline's x, its weights the
        # headline's, and without a capacity the routing of a prefix of the
        # tokens is that prefix's)
        y_ref, _ = oracle_reference(H, dcfg.T)
        result["decode_t64"] = {"ms_per_step": dms, "ms_per_step_graph_replay": dms_graph,
                                "tokens_per_s": dcfg.T / (dms * 1e-3),
                                "touched_experts": touched, "weight_bytes": wbytes,
                                "hbm_gbs": wbytes / (dms * 1e-3) / 1e9,
                                "hbm_frac": wbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                "parity": parity_report(dcfg, yd, y_ref)}
        log(f"decode {dms:.3f} ms/step")
        del D_, graph

    # ---- CPU oracle baseline on a bounded sample; its last run's y is the
    # parity reference of the timed run
    if not args.no_cpu_baseline:
        log(f"cpu baseline on {args.cpu_tokens} tokens")
        rec, y_ref, n_tok = cpu_baseline(H, args.cpu_tokens, args.cpu_repeats)
        result["cpu_baseline"] = rec
        result["parity"] = parity_report(cfg, y_gpu[:n_tok], y_ref)
        result["parity"]["what"] = ("max-abs error / RMS of the timed run's y against the "
                                    "oracle's float64 y")
        if n_tok < cfg.T:
            result["parity"]["note"] = "the oracle's routing of the first tokens only"
    else:
        result["cpu_baseline"] = None
    del H
    torch.cuda.empty_cache()

    # ---- the other workloads: step time against each one's binding floor
    if not args.no_sub and args.workload == "mixtral":
        subs = {}
        for name in SUB_WORKLOADS:
            subs[name] = sub_record(name, args.sub_steps, 3,
                                    parity=name in ("tiny", "capacity_skew"))
            torch.cuda.empty_cache()
        result["workloads"] = subs

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
