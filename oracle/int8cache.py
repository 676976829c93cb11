"""INT8 KV-cache quantization (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Summary] Inference lists "INT8 KV-cache quantization" among the single-GPU
optimisations; [News] and [Deploy] mention INT8 for the RTX 4090 path.  The
scheme is not given.  Reading taken: each (head, token) row of 128 values is
stored as 128 int8 codes q and one power-of-two scale 2^e (e an int8):

    e = the smallest integer with max_d |x_d| <= 127 * 2^e   (0 for a zero row,
        at least -127),
    q_d = x_d / 2^e rounded to the nearest integer, ties to even,

and the cached value is q_d * 2^e.  |q| <= 127 has at most 7 significant
bits, so q * 2^e is exactly representable in bf16: attention over the
dequantized cache is plain attention over those values, which the attention
oracle computes as it is.  The decision (the rounding of x / 2^e, an exact
power-of-two division) is taken in binary floating point on both sides.

Pins: tests/test_oracle_int8cache.py (hand-worked rows, ties, exact
round trips of representable rows, the half-step error bound, the code range
of the row maximum).
"""
from __future__ import annotations

import numpy as np


def row_exponents(x) -> np.ndarray:
    """e per row (last axis of x), int64."""
    amax = np.abs(np.asarray(x, np.float64)).max(axis=-1)
    m, k = np.frexp(amax)                 # amax = m * 2^k, m in [0.5, 1)
    e = k.astype(np.int64) - 7            # amax / 2^e = 128 m in [64, 128)
    e = np.where(128.0 * m > 127.0, e + 1, e)
    e = np.where(amax == 0.0, 0, e)
    return np.maximum(e, -127)


def quantize_rows(x):
    """(q int8 [..., 128], e int8 [...]) for rows x [..., 128]."""
    x = np.asarray(x, np.float64)
    e = row_exponents(x)
    q = np.rint(x / np.exp2(e.astype(np.float64))[..., None])   # rint: ties to even
    return q.astype(np.int8), e.astype(np.int8)


def dequantize_rows(q, e) -> np.ndarray:
    """q * 2^e in float64 (exact)."""
    return np.asarray(q, np.float64) * np.exp2(np.asarray(e, np.float64))[..., None]
