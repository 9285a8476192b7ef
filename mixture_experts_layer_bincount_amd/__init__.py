"""Thin Python binding of the MI355X MoE layer library (libmoe_mi355x.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions take torch tensors that live on the current HIP device
and enqueue work on torch's current stream; they raise MoEError on a non-OK
status.  There is no fallback: if the library is missing, importing this
package fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python mixture_experts_layer_bincount_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

DT_F32, DT_BF16, DT_FP8_E4M3, DT_INT8, DT_INT4 = 0, 1, 2, 3, 4
LINEAR_BIAS, SWIGLU = 0, 1
OVERFLOW_DROP, OVERFLOW_REROUTE, OVERFLOW_SHARED = 0, 1, 2
OVERFLOW = {"drop": OVERFLOW_DROP, "reroute": OVERFLOW_REROUTE, "shared": OVERFLOW_SHARED}
COMBINE_AUTO, COMBINE_GROUPED, COMBINE_FUSED = 0, 1, 2
COMBINE = {"auto": COMBINE_AUTO, "grouped": COMBINE_GROUPED, "fused": COMBINE_FUSED}
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_HIP"}

EXPORTS = ("moe_capacity", "moe_workspace_bytes", "moe_router_packed_bytes", "moe_pack_router",
           "moe_route", "moe_route_from_logits",
           "moe_reroute", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward",
           "moe_forward_noalloc",
           "moe_load_imbalance", "moe_lpt_pack", "moe_eplb_plan", "moe_timing_enable",
           "moe_timing_collect",
           "moe_timing_stage_name", "moe_last_error")


class MoEError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("has_shared", ctypes.c_int32), ("overflow", ctypes.c_int32),
                ("reroute_rounds", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("combine", ctypes.c_int32),
                ("hidden_split", ctypes.c_int32), ("router_packed", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("W1", "W3", "W2", "s1", "s3", "s2", "W1s", "W3s", "W2s",
                 "s1s", "s3s", "s2s", "W", "b")]


_vp = ctypes.c_void_p
_P = ctypes.POINTER
_lib.moe_capacity.restype = ctypes.c_int
_lib.moe_capacity.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
_lib.moe_workspace_bytes.restype = ctypes.c_size_t
_lib.moe_workspace_bytes.argtypes = [_P(Shape)]
_lib.moe_router_packed_bytes.restype = ctypes.c_size_t
_lib.moe_router_packed_bytes.argtypes = [_P(Shape)]
_lib.moe_pack_router.restype = ctypes.c_int
_lib.moe_pack_router.argtypes = [_P(Shape), _vp, _vp, _vp]
_lib.moe_route.restype = ctypes.c_int
_lib.moe_route.argtypes = [_P(Shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.moe_route_from_logits.restype = ctypes.c_int
_lib.moe_route_from_logits.argtypes = [_P(Shape), _vp, _vp, _vp, _vp]
_lib.moe_reroute.restype = ctypes.c_int
_lib.moe_reroute.argtypes = [_P(Shape)] + [_vp] * 5
_lib.moe_dispatch.restype = ctypes.c_int
_lib.moe_dispatch.argtypes = [_P(Shape)] + [_vp] * 12
_lib.moe_expert_ffn.restype = ctypes.c_int
_lib.moe_expert_ffn.argtypes = [_P(Shape), _P(Weights)] + [_vp] * 8
_lib.moe_combine.restype = ctypes.c_int
_lib.moe_combine.argtypes = [_P(Shape)] + [_vp] * 5
_lib.moe_forward.restype = ctypes.c_int
_lib.moe_forward.argtypes = [_P(Shape), _vp, _vp, _vp, _P(Weights)] + [_vp] * 7
_lib.moe_forward_noalloc.restype = ctypes.c_int
_lib.moe_forward_noalloc.argtypes = [_P(Shape), _vp, _vp, _vp, _P(Weights)] + [_vp] * 6
_lib.moe_load_imbalance.restype = ctypes.c_double
_lib.moe_load_imbalance.argtypes = [_P(ctypes.c_int64), ctypes.c_int32]
_lib.moe_lpt_pack.restype = ctypes.c_int
_lib.moe_lpt_pack.argtypes = [_P(ctypes.c_int64), ctypes.c_int32, ctypes.c_int32,
                              _P(ctypes.c_int32), _P(ctypes.c_int64)]
_lib.moe_eplb_plan.restype = ctypes.c_int
_lib.moe_eplb_plan.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp,
                               _vp, _vp]
_lib.moe_timing_enable.restype = ctypes.c_int
_lib.moe_timing_enable.argtypes = [ctypes.c_int]
_lib.moe_timing_collect.restype = ctypes.c_int
_lib.moe_timing_collect.argtypes = [_P(ctypes.c_double), ctypes.c_int, _P(ctypes.c_int)]
_lib.moe_timing_stage_name.restype = ctypes.c_char_p
_lib.moe_timing_stage_name.argtypes = [ctypes.c_int]
_lib.moe_last_error.restype = ctypes.c_char_p
_lib.moe_last_error.argtypes = []


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return t  # an integer address
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    if isinstance(stream, int):
        return stream  # a raw hipStream_t handle (0 = default stream)
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(st):
    if st != 0:
        raise MoEError(st, moe_last_error())


def make_shape(T, d, E, top_k, d_ff=0, capacity=-1, act_dtype=DT_BF16, w_dtype=DT_BF16,
               kind=SWIGLU, has_shared=False, overflow=OVERFLOW_DROP, reroute_rounds=0,
               n_groups=0, topk_groups=0, combine=COMBINE_AUTO, hidden_split=False,
               router_packed=False) -> Shape:
    """overflow: OVERFLOW_* or its name ("drop", "reroute", "shared").
    n_groups / topk_groups: group-limited routing (0 = off).
    combine: COMBINE_* or its name ("auto", "grouped", "fused").
    hidden_split: keep the SwiGLU hidden activation as two bf16 terms.
    router_packed: W_g arguments are moe_pack_router's buffer."""
    if isinstance(overflow, str):
        overflow = OVERFLOW[overflow]
    if isinstance(combine, str):
        combine = COMBINE[combine]
    return Shape(int(T), int(d), int(E), int(top_k), int(d_ff), int(capacity), int(act_dtype),
                 int(w_dtype), int(kind), int(bool(has_shared)), int(overflow),
                 int(reroute_rounds), int(n_groups), int(topk_groups), int(combine),
                 int(bool(hidden_split)), int(bool(router_packed)))


def make_weights(**tensors) -> Weights:
    w = Weights()
    for k, v in tensors.items():
        setattr(w, k, _ptr(v))
    w._keep = tensors  # keep the tensors alive with the struct
    return w


# ---------------------------------------------------------------- host entry points
def moe_capacity(T, E, k, cf) -> int:
    return int(_lib.moe_capacity(int(T), int(E), int(k), float(cf if cf is not None else 0.0)))


def moe_workspace_bytes(shape: Shape) -> int:
    return int(_lib.moe_workspace_bytes(ctypes.byref(shape)))


def moe_load_imbalance(load) -> float:
    arr = (ctypes.c_int64 * len(load))(*[int(v) for v in load])
    return float(_lib.moe_load_imbalance(arr, len(load)))


def moe_lpt_pack(load, D):
    E = len(load)
    arr = (ctypes.c_int64 * E)(*[int(v) for v in load])
    assign = (ctypes.c_int32 * E)()
    bins = (ctypes.c_int64 * D)()
    _check(_lib.moe_lpt_pack(arr, E, D, assign, bins))
    return list(assign), list(bins)


def moe_timing_enable(on: bool) -> None:
    _check(_lib.moe_timing_enable(1 if on else 0))


def moe_timing_collect():
    """{stage name: summed ms since the last collect}, number of timed calls."""
    ms = (ctypes.c_double * 16)()
    calls = ctypes.c_int(0)
    n = _lib.moe_timing_collect(ms, 16, ctypes.byref(calls))
    return {moe_timing_stage_name(i): ms[i] for i in range(n)}, calls.value


def moe_timing_stage_name(i: int) -> str:
    return _lib.moe_timing_stage_name(i).decode()


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


# ---------------------------------------------------------------- device entry points
def workspace(shape: Shape, device="cuda") -> torch.Tensor:
    n = moe_workspace_bytes(shape)
    if n == 0:
        raise MoEError(1, moe_last_error() or "invalid shape")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_router_packed_bytes(shape: Shape) -> int:
    return int(_lib.moe_router_packed_bytes(ctypes.byref(shape)))


def moe_pack_router(shape, W_g, packed, stream=None):
    _check(_lib.moe_pack_router(ctypes.byref(shape), _ptr(W_g), _ptr(packed), _stream(stream)))


def moe_route(shape, x, W_g, b_g, logits, topk_idx, topk_w, ws, stream=None):
    _check(_lib.moe_route(ctypes.byref(shape), _ptr(x), _ptr(W_g), _ptr(b_g), _ptr(logits),
                          _ptr(topk_idx), _ptr(topk_w), _ptr(ws), _stream(stream)))


def moe_route_from_logits(shape, logits, topk_idx, topk_w, stream=None):
    _check(_lib.moe_route_from_logits(ctypes.byref(shape), _ptr(logits), _ptr(topk_idx),
                                      _ptr(topk_w), _stream(stream)))


def moe_reroute(shape, logits, topk_idx, final_idx, ws, stream=None):
    _check(_lib.moe_reroute(ctypes.byref(shape), _ptr(logits), _ptr(topk_idx), _ptr(final_idx),
                            _ptr(ws), _stream(stream)))


def moe_dispatch(shape, topk_idx, topk_w, x, counts, offsets, keep, perm_token, perm_w,
                 slot_pos, x_perm, ws, stream=None):
    _check(_lib.moe_dispatch(ctypes.byref(shape), _ptr(topk_idx), _ptr(topk_w), _ptr(x),
                             _ptr(counts), _ptr(offsets), _ptr(keep), _ptr(perm_token),
                             _ptr(perm_w), _ptr(slot_pos), _ptr(x_perm), _ptr(ws),
                             _stream(stream)))


def moe_expert_ffn(shape, weights, x, offsets, perm_token, perm_w, y_perm, y, ws, stream=None):
    _check(_lib.moe_expert_ffn(ctypes.byref(shape), ctypes.byref(weights), _ptr(x),
                               _ptr(offsets), _ptr(perm_token), _ptr(perm_w), _ptr(y_perm),
                               _ptr(y), _ptr(ws), _stream(stream)))


def moe_combine(shape, y_perm, slot_pos, topk_w, y, stream=None):
    _check(_lib.moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(slot_pos), _ptr(topk_w),
                            _ptr(y), _stream(stream)))


def moe_eplb_plan(counts, D, extra, replicas, slot_device, slot_load, device_load, stream=None):
    """Device-side replication + placement from the int32 counts tensor [E]."""
    _check(_lib.moe_eplb_plan(_ptr(counts), int(counts.numel()), int(D), int(extra),
                              _ptr(replicas), _ptr(slot_device), _ptr(slot_load),
                              _ptr(device_load), _stream(stream)))


def moe_forward(shape, x, W_g, b_g, weights, y, topk_idx, topk_w, counts, offsets, ws,
                stream=None):
    _check(_lib.moe_forward(ctypes.byref(shape), _ptr(x), _ptr(W_g), _ptr(b_g),
                            ctypes.byref(weights), _ptr(y), _ptr(topk_idx), _ptr(topk_w),
                            _ptr(counts), _ptr(offsets), _ptr(ws), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(shape, x, W_g, b_g, weights, y, topk_idx, topk_w, counts, offsets,
                        stream=None):
    _check(_lib.moe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(W_g), _ptr(b_g),
                                    ctypes.byref(weights), _ptr(y), _ptr(topk_idx),
                                    _ptr(topk_w), _ptr(counts), _ptr(offsets),
                                    _stream(stream)))


from .layer import MoELayer  # noqa: E402,F401
