"""Seeded input generation for the MoE layer workloads.

Recipe (one `numpy.random.SeedSequence(cfg.seed)` per workload; children are
spawned once, in a fixed order, so any expert's weights can be regenerated on
their own and in parallel):

  child 0      x[T, d]          N(0, 1)
  child 1      W_g[d, E] fp32   N(0, 1/d)          (router, stored [in, out])
  child 2      b_g[E]           unused draw slot (the skewed workload's bias is
                                 the closed form 1.5*ln(1/(e+1)), not random)
  per expert e (children 3 + 3e .. 5 + 3e):
    SwiGLU:    W1[e][d_ff, d] N(0, 1/d), W3[e][d_ff, d] N(0, 1/d),
               W2[e][d, d_ff] N(0, 1/d_ff)
    Linear:    W[e][d, d] N(0, 1/d), b[e][d] N(0, 0.01) (std 0.1), third slot unused
  shared expert (children 3 + 3E .. 5 + 3E): W1s, W3s, W2s as for SwiGLU

Expert weights are stored output-major ([out, in], the nn.Linear layout and
the merged [num_experts*ffn_dim, hidden_dim] layout of the iopenshare page's
MergedExpertLayer, §5.2), so the reduction dimension is contiguous.

Values are drawn as float32 standard normals times the std, then rounded to
bfloat16 with round-to-nearest-even when the workload is bf16.  bf16 arrays
are numpy uint16 bit patterns.

The fp8 workload quantises the bf16 weights to OCP FP8 E4M3 with one fp32
scale per group of 128 output features: s = amax(group)/448 and
code = RNE(w/s), via torch's float8_e4m3fn conversion.  The int8 workload
uses symmetric int8 codes with the same grouping: s = amax(group)/127 and
code = RNE(w/s) in float32, clipped to [-127, 127].  The int4 workload does
the same with s = amax(group)/7 and codes clipped to [-7, 7], stored as
offset-binary nibbles c = n + 8: each group of 8 consecutive inputs takes 4
bytes, byte b holding input b in its low nibble and input b + 4 in its high
nibble, in the one-field structured dtype INT4X2.  This is weight preparation of the input,
not part of the layer.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from .configs import CONFIGS, MoEConfig

FP8_GROUP = 128
FP8_MAX = 448.0
INT8_MAX = 127.0
INT4_MAX = 7.0
# packed int4 codes: a one-field structured byte, so they are told apart from
# int8 or fp8 codes by their dtype
INT4X2 = np.dtype([("int4x2", np.uint8)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (RNE); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _normal(seed_seq, shape, std) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def _quant_fp8_rows(w_bf16: np.ndarray):
    """Quantise a [out, in] bf16 matrix to e4m3 codes with per-128-row scales."""
    import torch
    w = torch.from_numpy(bf16_bits_to_f32(w_bf16))
    out, inn = w.shape
    g = w.view(out // FP8_GROUP, FP8_GROUP, inn)
    amax = g.abs().amax(dim=(1, 2)).clamp_min(1e-30)
    s = (amax / FP8_MAX).to(torch.float32)
    q = (g / s[:, None, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(out, inn)
    return codes.numpy().copy(), s.numpy().copy()


def _quant_int8_rows(w_bf16: np.ndarray):
    """Quantise a [out, in] bf16 matrix to symmetric int8 codes with
    per-128-row scales."""
    w = bf16_bits_to_f32(w_bf16)
    out, inn = w.shape
    g = w.reshape(out // FP8_GROUP, FP8_GROUP, inn)
    amax = np.maximum(np.abs(g).max(axis=(1, 2)), np.float32(1e-30))
    s = (amax / np.float32(INT8_MAX)).astype(np.float32)
    q = np.clip(np.rint(g / s[:, None, None]), -INT8_MAX, INT8_MAX).astype(np.int8)
    return q.reshape(out, inn), s


def _quant_int4_rows(w_bf16: np.ndarray):
    """Quantise a [out, in] bf16 matrix to symmetric int4 codes with
    per-128-row scales, packed two per byte ([out, in/2], INT4X2)."""
    w = bf16_bits_to_f32(w_bf16)
    out, inn = w.shape
    g = w.reshape(out // FP8_GROUP, FP8_GROUP, inn)
    amax = np.maximum(np.abs(g).max(axis=(1, 2)), np.float32(1e-30))
    s = (amax / np.float32(INT4_MAX)).astype(np.float32)
    q = np.clip(np.rint(g / s[:, None, None]), -INT4_MAX, INT4_MAX).astype(np.int16)
    c = (q.reshape(out, inn // 8, 8) + 8).astype(np.uint8)      # offset binary
    packed = (c[:, :, 0:4] | (c[:, :, 4:8] << np.uint8(4))).reshape(out, inn // 2)
    return np.ascontiguousarray(packed).view(INT4X2), s


class Workload:
    """Lazily generated inputs of one workload."""

    def __init__(self, cfg: MoEConfig | str):
        if isinstance(cfg, str):
            cfg = CONFIGS[cfg]
        self.cfg = cfg
        wcfg = CONFIGS[cfg.w_from] if cfg.w_from else cfg
        self._wcfg = wcfg
        n_children = 3 + 3 * wcfg.E + 3
        self._children = np.random.SeedSequence(wcfg.seed).spawn(n_children)
        self._x = None

    # ---- activations and router -------------------------------------------------
    def x(self) -> np.ndarray:
        """x[T, d]: float32 for f32 workloads, bf16 bits (uint16) otherwise."""
        if self._x is None:
            c = self.cfg
            if c.x_from:
                src = Workload(CONFIGS[c.x_from])
                self._x = np.ascontiguousarray(src.x()[: c.T])
            else:
                a = _normal(self._children[0], (c.T, c.d), 1.0)
                self._x = a if c.act == "f32" else f32_to_bf16_bits(a)
        return self._x

    def W_g(self) -> np.ndarray:
        c = self._wcfg
        return _normal(self._children[1], (c.d, c.E), 1.0 / np.sqrt(c.d))

    def b_g(self):
        c = self._wcfg
        if c.router_bias is None:
            return None
        if c.router_bias == "zipf1.5":
            e = np.arange(c.E, dtype=np.float64)
            return (1.5 * np.log(1.0 / (e + 1.0))).astype(np.float32)
        raise ValueError(c.router_bias)

    # ---- experts -------------------------------------------------------------------
    def expert(self, e: int) -> dict:
        """Weights of routed expert e in the workload's weight dtype."""
        c = self._wcfg
        ch = self._children[3 + 3 * e: 6 + 3 * e]
        if c.kind == "linear_bias":
            W = _normal(ch[0], (c.d, c.d), 1.0 / np.sqrt(c.d))
            b = _normal(ch[1], (c.d,), 0.1)
            return {"W": W, "b": b}
        return self._swiglu(ch, c)

    def shared(self):
        c = self._wcfg
        if not c.shared:
            return None
        ch = self._children[3 + 3 * c.E: 6 + 3 * c.E]
        return self._swiglu(ch, c)

    def _swiglu(self, ch, c) -> dict:
        W1 = f32_to_bf16_bits(_normal(ch[0], (c.d_ff, c.d), 1.0 / np.sqrt(c.d)))
        W3 = f32_to_bf16_bits(_normal(ch[1], (c.d_ff, c.d), 1.0 / np.sqrt(c.d)))
        W2 = f32_to_bf16_bits(_normal(ch[2], (c.d, c.d_ff), 1.0 / np.sqrt(c.d_ff)))
        if self.cfg.w == "fp8_e4m3":
            q1, s1 = _quant_fp8_rows(W1)
            q3, s3 = _quant_fp8_rows(W3)
            q2, s2 = _quant_fp8_rows(W2)
            return {"W1": q1, "W3": q3, "W2": q2, "s1": s1, "s3": s3, "s2": s2}
        if self.cfg.w in ("int8", "int4"):
            quant = _quant_int8_rows if self.cfg.w == "int8" else _quant_int4_rows
            q1, s1 = quant(W1)
            q3, s3 = quant(W3)
            q2, s2 = quant(W2)
            return {"W1": q1, "W3": q3, "W2": q2, "s1": s1, "s3": s3, "s2": s2}
        return {"W1": W1, "W3": W3, "W2": W2}

    def experts_parallel(self, es, fn, workers=None):
        """Generate experts `es` on a thread pool and hand each to fn(e, weights).

        numpy's generators and ufuncs release the GIL on large fills, so the
        threads run concurrently.  fn runs on the calling thread, in order of e.
        """
        es = list(es)
        workers = workers or min(16, len(os.sched_getaffinity(0)))
        with cf.ThreadPoolExecutor(max_workers=workers) as pool:
            futs = {}
            it = iter(es)
            for e in it:
                futs[e] = pool.submit(self.expert, e)
                if len(futs) >= workers:
                    break
            pending = [e for e in es if e not in futs]
            for e in es:
                w = futs.pop(e).result()
                if pending:
                    e2 = pending.pop(0)
                    futs[e2] = pool.submit(self.expert, e2)
                fn(e, w)
