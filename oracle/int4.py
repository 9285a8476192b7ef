"""Symmetric int4 expert weights (oracle; test infrastructure only).

iopenshare "MoE 混合专家架构" §5.3 names INT4 quantisation of the expert
weights without fixing a format.  Read here as: codes in [-7, 7], two per byte
along the input (reduction) dimension, the code of the even input index in the
low nibble and each nibble a 4-bit two's-complement number; one float32 scale
per group of 128 output features (rows of the [out, in] matrix); weight =
code * scale.  A packed matrix is a numpy array of the one-field structured
dtype INT4X2 ([out, in/2] bytes), which tells it apart from int8 or fp8 codes.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
INT4X2 = np.dtype([("int4x2", np.uint8)])


def is_int4x2(a: np.ndarray) -> bool:
    return a.dtype.names == ("int4x2",)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """[out, in/2] packed bytes -> [out, in] int64 codes in [-8, 7]."""
    b = np.ascontiguousarray(packed).view(np.uint8).astype(np.int64)
    out, half = b.shape
    nib = np.empty((out, 2 * half), dtype=np.int64)
    nib[:, 0::2] = b & 0xF          # even input index: low nibble
    nib[:, 1::2] = b >> 4           # odd input index: high nibble
    return np.where(nib >= 8, nib - 16, nib)


def dequant_int4_rows(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[out, in/2] packed int4 codes -> [out, in] float64 weights, row r
    scaled by scales[r // 128].  Exact in float64."""
    codes = unpack_int4(packed).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), GROUP)[: codes.shape[0]]
    return codes * s[:, None]
