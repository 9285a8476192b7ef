"""OCP FP8 E4M3 decoding for the fp8-weight workload (oracle; test
infrastructure only).

The pages only mention INT8/INT4 weight quantisation (iopenshare §5.3); the fp8
run's format is the OCP 8-bit floating point E4M3 encoding: sign, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
(m/8 * 2^-6); no infinities; S.1111.111 is NaN; the largest finite value is
448 (S.1111.110).  Weights are code * scale with one float32 scale per group
of 128 output features (rows of the [out, in] matrix).
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode_table() -> np.ndarray:
    return _TABLE.copy()


def dequant_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[out, in] codes -> float64 weights, row r scaled by scales[r // 128].
    Exact: a 4-bit significand times a float32 fits in float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    vals = _TABLE[codes]
    s = np.repeat(np.asarray(scales, dtype=np.float64), GROUP)[: codes.shape[0]]
    return vals * s[:, None]
