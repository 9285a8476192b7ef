"""Symmetric int8 expert weights (oracle; test infrastructure only).

iopenshare "MoE 混合专家架构" §5.3 names INT8/INT4 quantisation of the expert
weights without fixing a format.  Read here as: symmetric int8 codes in
[-127, 127] and one float32 scale per group of 128 output features (rows of
the [out, in] matrix), weight = code * scale -- the same grouping as the fp8
run, so the scale is constant along the reduction.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def dequant_int8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[out, in] int8 codes -> float64 weights, row r scaled by scales[r // 128].
    Exact: a code of at most 8 bits times a float32 fits in float64."""
    codes = np.asarray(codes, dtype=np.int8).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), GROUP)[: codes.shape[0]]
    return codes * s[:, None]
