"""Pins of the INT8 KV-cache quantizer (oracle/int8cache.py).

The reading (per (head, token) row: int8 codes and one power-of-two scale,
the smallest that keeps every code within +-127, round half to even) is
checked against rows worked out by hand, the tie rule, exact round trips of
values the format can hold, the half-step error bound and the range of the
row maximum's code.
"""
import numpy as np
import pytest

from oracle.int8cache import dequantize_rows, quantize_rows, row_exponents
from segment_causal_masked_amd.workloads import randn


def row(*vals):
    x = np.zeros(128)
    x[:len(vals)] = vals
    return x


def test_hand_worked_rows():
    # max 1.0: 1.0 / 2^-6 = 64 <= 127, 1.0 / 2^-7 = 128 > 127  ->  e = -6
    q, e = quantize_rows(row(1.0, -0.5, 0.3, 0.0078125))
    assert int(e) == -6
    assert list(q[:4]) == [64, -32, 19, 0]          # 0.3 * 64 = 19.2; 0.5 -> 0 (tie, even)
    # max 127 * 2^-6 = 1.984375: exactly 127 at e = -6
    q, e = quantize_rows(row(1.984375, -1.0))
    assert int(e) == -6 and list(q[:2]) == [127, -64]
    # max 255 / 128 = 1.9921875: 127.5 at e = -6 is too large -> e = -5, 63.75 -> 64
    q, e = quantize_rows(row(1.9921875, 0.25))
    assert int(e) == -5 and list(q[:2]) == [64, 8]
    # max 3.0: 3 / 2^-5 = 96 -> e = -5
    q, e = quantize_rows(row(-3.0, 2.0, 0.046875))
    assert int(e) == -5 and list(q[:3]) == [-96, 64, 2]   # 0.046875 * 32 = 1.5 -> 2 (tie, even)
    # a zero row
    q, e = quantize_rows(np.zeros(128))
    assert int(e) == 0 and not q.any()


def test_ties_round_to_even():
    # max 1.0 fixes e = -6; x = (k + 0.5) / 64 lies halfway between codes
    vals = [(k + 0.5) / 64 for k in range(-6, 6)]
    q, e = quantize_rows(row(1.0, *vals))
    assert int(e) == -6
    want = [k if k % 2 == 0 else k + 1 for k in range(-6, 6)]
    assert list(q[1:13]) == want


def test_representable_rows_round_trip_exactly():
    g = np.random.default_rng(3)
    for _ in range(50):
        e = int(g.integers(-20, 10))
        q = g.integers(-127, 128, size=128)
        q[int(g.integers(0, 128))] = int(g.choice([-127, 127, 64, -64, 100]))
        x = q * 2.0 ** e
        q2, e2 = quantize_rows(x)
        np.testing.assert_array_equal(dequantize_rows(q2, e2), x)


def test_error_bound_and_code_range():
    x = randn((64, 16, 128), 77)
    q, e = quantize_rows(x)
    deq = dequantize_rows(q, e)
    step = np.exp2(e.astype(np.float64))[..., None]
    assert np.all(np.abs(deq - x) <= step / 2)
    amax_code = np.abs(q.astype(np.int64)).max(axis=-1)
    assert np.all((amax_code >= 64) & (amax_code <= 127))
    assert np.all(np.abs(q.astype(np.int64)) <= 127)
    # the next smaller scale would overflow the codes
    assert np.all(np.abs(x).max(axis=-1) / np.exp2(e.astype(np.float64) - 1) > 127)


def test_dequantized_values_are_bf16_exact():
    x = randn((32, 4, 128), 78)
    deq = dequantize_rows(*quantize_rows(x)).astype(np.float32)
    bits = deq.view(np.uint32)
    assert not np.any(bits & 0xFFFF)            # nothing below the bf16 mantissa


@pytest.mark.parametrize("scale", [2.0 ** -100, 2.0 ** 40])
def test_exponent_follows_magnitude(scale):
    x = randn((8, 128), 79) * scale
    e = row_exponents(x)
    e1 = row_exponents(x / scale)
    np.testing.assert_array_equal(e, e1 + int(np.log2(scale)))
