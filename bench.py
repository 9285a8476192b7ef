#!/usr/bin/env python3
"""Benchmark of the MoE FFN layer forward pass on one MI355X.

Workload: the Mixtral-shaped layer (T=4096 tokens, d=4096, E=8 experts,
top-2, SwiGLU experts with d_ff=14336, bf16 activations and weights, fp32
router, no capacity limit), synthetic seeded inputs resident in HBM before
the timed region.  One step = one full moe_forward (router, top-k, dispatch,
grouped gate/up GEMM + SwiGLU, grouped down GEMM + fused combine).

Prints one JSON line.  Also reported: the decode-shaped layer (the same
weights, T=64) in HBM GB/s over the touched expert weights, the dominant
kernel against its roofline (timed with HIP events on the launch stream),
and the CPU oracle timed on a bounded sample of the same workload.
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


def _traffic_from_profile(kernel_src: str, launches_bytes_key: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None when the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "gate_up_swiglu_mixtral_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(kernel_src, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()
    if rec.get("kernel_source_sha256") != h:
        return None
    return rec.get(launches_bytes_key)


def cpu_baseline(wl, host_experts, n_tokens: int, repeats: int, overflow="drop",
                 rounds=0, groups=0, topk_groups=0) -> dict:
    """The oracle as it stands, on the first n_tokens tokens of the workload
    (routing, dispatch, masked per-expert loop, combine; float64), run
    `repeats` times."""
    import oracle
    c = wl.cfg
    n_tokens = min(n_tokens, c.T)
    x = wl.x()[:n_tokens]
    W_g = wl.W_g()
    t0 = time.perf_counter()
    for _ in range(repeats):
        oracle.forward(x, W_g, wl.b_g(), c.k, c.E, lambda e: host_experts[e], kind=c.kind,
                       C=oracle.capacity(n_tokens, c.E, c.k, c.cf),
                       shared=wl.shared if c.shared else None, overflow=overflow, rounds=rounds,
                       groups=groups, topk_groups=topk_groups)
    dt = time.perf_counter() - t0
    return {"value": n_tokens * repeats / dt, "unit": "tokens/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"first {n_tokens} of the {c.T} tokens of the {c.name} workload, whole "
                      f"layer (router, top-k, bincount, dispatch, masked per-expert loop, "
                      f"combine) in float64 NumPy, {repeats} runs; {dt:.1f} s on {_cpu_model()}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
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
    from moe_synth import Workload, get_config
    from moe_synth.device import to_device

    torch.cuda.set_device(0)
    cfg = get_config(args.workload)
    wl = Workload(cfg)
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    host_experts = {}
    wl.experts_parallel(range(cfg.E), lambda e, w: host_experts.__setitem__(e, w))
    dev_w = {}
    for name in host_experts[0]:
        dev_w[name] = to_device(np.stack([host_experts[e][name] for e in range(cfg.E)]), "cuda")
    sh = wl.shared()
    if sh is not None:
        for name, a in sh.items():
            dev_w[name + "s"] = to_device(a, "cuda")
    x = to_device(wl.x(), "cuda")
    W_g = to_device(wl.W_g(), "cuda")
    b = wl.b_g()
    b_g = to_device(b, "cuda") if b is not None else None
    cap = moe.moe_capacity(cfg.T, cfg.E, cfg.k, cfg.cf) if cfg.cf else -1
    rounds = args.rounds if args.overflow == "reroute" else 0
    layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, W_g=W_g, b_g=b_g, weights=dev_w,
                         capacity=cap, kind=cfg.kind, w_dtype=cfg.w, has_shared=cfg.shared,
                         overflow=args.overflow, reroute_rounds=rounds, n_groups=args.groups,
                         topk_groups=args.topk_groups)
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer(x)
    torch.cuda.synchronize()

    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- timed region: K steps, stage events recorded on the launch stream
    moe.moe_timing_enable(True)
    moe.moe_timing_collect()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        layer(x)
    ev1.record()
    torch.cuda.synchronize()
    stage_ms, calls = moe.moe_timing_collect()
    moe.moe_timing_enable(False)
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {args.steps} steps, {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    kept = int(layer.offsets[-1].item())
    counts = layer.counts.cpu().tolist()
    flops_gate_up = 2.0 * kept * cfg.d * 2 * cfg.d_ff
    flops_down = 2.0 * kept * cfg.d_ff * cfg.d
    flops_ffn = flops_gate_up + flops_down
    gu_ms = stage_ms["gate_up_swiglu"] / max(calls, 1)
    dn_ms = stage_ms["down_combine"] / max(calls, 1)
    achieved = flops_gate_up / (gu_ms * 1e-3) / 1e12
    gemm_src = os.path.join(ROOT, "mixture_experts_layer_bincount_amd", "csrc", "expert_gemm.hip")
    traffic = _traffic_from_profile(gemm_src, "hbm_bytes_per_launch")
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
                   "capacity": cap, "overflow": args.overflow, "reroute_rounds": rounds,
                   "groups": args.groups, "topk_groups": args.topk_groups,
                   "global_batch": cfg.T, "parallelism": "none (1 GPU)"},
        "layer_mfma_frac": flops_ffn / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "layer_tflops": flops_ffn / (ms_per_step * 1e-3) / 1e12,
        "stage_ms": stages,
        "counts": counts,
        "roofline": {"kernel": "grouped gate/up GEMM + SwiGLU (grouped_gemm_dma_kernel<GATEUP>)",
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "algorithmic_per_launch": f"{flops_gate_up:.4e} FLOP = 2*{kept} rows*"
                                               f"{cfg.d}*2*{cfg.d_ff}",
                     "avg_launch_ms": gu_ms,
                     "down_combine": {"avg_launch_ms": dn_ms,
                                      "tflops": flops_down / (dn_ms * 1e-3) / 1e12}},
    }

    # ---- load statistics of this step's routing (tutorial §4.2 / §4.3: the
    # imbalance max/(min + 1e-6) and the LPT packing of the expert loads onto
    # 8 devices, by the library's host functions), on the raw counts and on
    # the kept (capacity-limited) rows
    kept_rows = np.diff(layer.offsets.cpu().numpy()).tolist()
    stats = {}
    for name, load in (("counts", counts), ("kept", kept_rows)):
        _, bins = moe.moe_lpt_pack(load, 8)
        stats[name] = {"imbalance": moe.moe_load_imbalance(load),
                       "max_over_mean": max(load) / (sum(load) / len(load)),
                       "empty_experts": int(sum(1 for v in load if v == 0)),
                       "lpt_8_bins": bins,
                       "lpt_8_max_over_mean": max(bins) / (sum(bins) / len(bins))}
    result["load_stats"] = stats

    # ---- weight stream: the bytes of the experts this step touched (codes
    # and scales in the workload's weight format, the shared expert included)
    # against the step time and against the two FFN stages
    if cfg.kind == "swiglu":
        wbits = {"bf16": 16, "fp8_e4m3": 8, "int8": 8, "int4": 4}[cfg.w]
        per_expert = 3 * cfg.d * cfg.d_ff * wbits // 8
        if wbits != 16:
            per_expert += 4 * (2 * cfg.d_ff + cfg.d) // 128
        n_exp = sum(1 for v in kept_rows if v > 0) + (1 if cfg.shared else 0)
        wb = n_exp * per_expert
        ffn_ms = gu_ms + dn_ms
        result["weight_stream"] = {
            "experts": n_exp, "bytes": wb,
            "gbs_over_step": wb / (ms_per_step * 1e-3) / 1e9,
            "hbm_frac_over_step": wb / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "gbs_over_ffn_stages": wb / (ffn_ms * 1e-3) / 1e9}

    # ---- online EPLB on the device: replicas + placement onto 8 devices from
    # this step's counts (still on the device), E/8 extra replicas
    D, extra = 8, max(1, cfg.E // 8)
    reps = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    sdev = torch.empty(cfg.E + extra, dtype=torch.int32, device="cuda")
    sload = torch.empty(cfg.E + extra, dtype=torch.int32, device="cuda")
    dload = torch.empty(D, dtype=torch.int64, device="cuda")
    for _ in range(3):
        moe.moe_eplb_plan(layer.counts, D, extra, reps, sdev, sload, dload)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        moe.moe_eplb_plan(layer.counts, D, extra, reps, sdev, sload, dload)
    e1.record()
    torch.cuda.synchronize()
    dl = dload.cpu().numpy()
    result["eplb_plan"] = {"devices": D, "extra_replicas": extra,
                           "us_per_plan": e0.elapsed_time(e1) / 20 * 1e3,
                           "device_load_max_over_mean": float(dl.max() / dl.mean()),
                           "without_replicas_max_over_mean": stats["counts"]["lpt_8_max_over_mean"]}

    # ---- decode-shaped layer: the same weights, the first 64 tokens
    if not args.no_decode and cfg.name == "mixtral":
        dcfg = get_config("decode")
        xd = x[: dcfg.T].contiguous()
        dl = moe.MoELayer(dcfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, W_g=W_g, b_g=b_g,
                          weights=dev_w, kind=cfg.kind, w_dtype=cfg.w)
        for _ in range(3):
            dl(xd)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.decode_steps):
            dl(xd)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.decode_steps
        # the same decode step replayed from a captured HIP graph (no
        # per-kernel launch cost on the host side)
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            dl(xd)
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dl(xd)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.decode_steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        dms_graph = e0.elapsed_time(e1) / args.decode_steps
        dcounts = dl.counts.cpu().numpy()
        touched = int((dcounts > 0).sum())
        wbytes = touched * 3 * cfg.d * cfg.d_ff * 2
        result["decode_t64"] = {"ms_per_step": dms, "ms_per_step_graph_replay": dms_graph,
                                "tokens_per_s": dcfg.T / (dms * 1e-3),
                                "touched_experts": touched,
                                "hbm_gbs": wbytes / (dms * 1e-3) / 1e9,
                                "hbm_frac": wbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        print(f"[bench] decode {dms:.3f} ms/step", file=sys.stderr, flush=True)

    # ---- CPU oracle baseline on a bounded sample
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, host_experts, args.cpu_tokens, args.cpu_repeats,
                                              args.overflow, rounds, args.groups,
                                              args.topk_groups)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
