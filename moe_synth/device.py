"""Upload a generated workload to the HIP device as torch tensors (plumbing)."""
from __future__ import annotations

import numpy as np
import torch

from .gen import Workload


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """numpy -> torch on `device`; uint16 arrays become bfloat16 tensors,
    packed int4 (one-field structured bytes) uint8 tensors."""
    if a.dtype.names:
        a = np.ascontiguousarray(a).view(np.uint8)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(wl: Workload, device="cuda", workers=None, keep_host=None):
    """Returns dict(x, W_g, b_g, weights) of device tensors; expert weights
    are stacked [E, out, in] (and scales [E, out/128]).  keep_host: a dict
    that receives each routed expert's host arrays (e -> dict), or None."""
    c = wl._wcfg
    dev = torch.device(device)
    out = {"x": to_device(wl.x(), dev), "W_g": to_device(wl.W_g(), dev)}
    b = wl.b_g()
    out["b_g"] = to_device(b, dev) if b is not None else None
    weights = {}
    if c.kind == "linear_bias":
        Ws, bs = [], []
        for e in range(c.E):
            w = wl.expert(e)
            Ws.append(w["W"])
            bs.append(w["b"])
            if keep_host is not None:
                keep_host[e] = w
        weights["W"] = to_device(np.stack(Ws), dev)
        weights["b"] = to_device(np.stack(bs), dev)
    else:
        first = wl.expert(0)
        for name, a in first.items():
            weights[name] = torch.empty((c.E,) + a.shape,
                                        dtype=to_device(a[:1] if a.ndim else a, "cpu").dtype, device=dev)

        def put(e, w):
            for name, a in w.items():
                weights[name][e].copy_(to_device(a, "cpu"), non_blocking=False)
            if keep_host is not None:
                keep_host[e] = w

        wl.experts_parallel(range(c.E), put, workers=workers)
        sh = wl.shared()
        if sh is not None:
            for name, a in sh.items():
                weights[name + "s"] = to_device(a, dev)
    out["weights"] = weights
    return out
