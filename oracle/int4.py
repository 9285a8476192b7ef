"""Symmetric int4 expert weights (oracle; test infrastructure only).

iopenshare "MoE 混合专家架构" §5.3 names INT4 quantisation of the expert
weights without fixing a format.  Read here as: integer codes n in [-7, 7]
(the format also holds -8), one float32 scale per group of 128 output
features (rows of the [out, in] matrix), weight = n * scale.  Storage: each
code is the 4-bit offset-binary number c = n + 8; along a weight row the
inputs form groups of 8 consecutive ones, each stored in 4 bytes, where byte b
(b = 0..3) holds the code of input 8g + b in its low nibble and the code of
input 8g + b + 4 in its high nibble.  A packed matrix is a numpy array of the
one-field structured dtype INT4X2 ([out, in/2] bytes), which tells it apart
from int8 or fp8 codes.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
ZERO = 8
INT4X2 = np.dtype([("int4x2", np.uint8)])


def is_int4x2(a: np.ndarray) -> bool:
    return a.dtype.names == ("int4x2",)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """[out, in/2] packed bytes -> [out, in] int64 integers n in [-8, 7]."""
    b = np.ascontiguousarray(packed).view(np.uint8).astype(np.int64)
    out, half = b.shape
    g = b.reshape(out, half // 4, 4)              # one 8-input group per 4 bytes
    n = np.empty((out, half // 4, 8), dtype=np.int64)
    n[:, :, 0:4] = (g & 0xF) - ZERO               # inputs 8g .. 8g+3: low nibbles
    n[:, :, 4:8] = (g >> 4) - ZERO                # inputs 8g+4 .. 8g+7: high nibbles
    return n.reshape(out, 2 * half)


def dequant_int4_rows(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[out, in/2] packed int4 codes -> [out, in] float64 weights, row r
    scaled by scales[r // 128].  Exact in float64."""
    codes = unpack_int4(packed).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), GROUP)[: codes.shape[0]]
    return codes * s[:, None]
