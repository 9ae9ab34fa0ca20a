"""Pins of the oracle's int8 weight quantizer (nanoinfer page, phase 6).

Each pin is something the page fixes or the arithmetic implies, chosen so that a
plausible slip fails one of them: rounding to even instead of away from zero,
adding 0.5 then truncating, a per-tensor scale, a [-128, 127] range, a sign
error, or a scale that is not max/127.
"""
import numpy as np

from oracle.numerics import f32_to_bf16_bits
from oracle.quant import dequantize, quantize_rows_int8, round_half_away


def test_ties_round_half_away_from_zero():
    # max 127 -> scale exactly 1, so each code is the rounded value itself
    w = np.array([[127.0, 62.5, -62.5, 0.5, -0.5, 1.5, 2.5, -2.5, 0.0, 126.5]], np.float32)
    q, s = quantize_rows_int8(w)
    assert s[0] == np.float32(1.0)
    assert q[0].tolist() == [127, 63, -63, 1, -1, 2, 3, -3, 0, 127]   # np.round would give 62, 0, 2


def test_just_below_half_rounds_down():
    # 0.5 - 2^-25: adding 0.5 in float32 rounds to 1.0, the exact rule keeps 0
    below = np.nextafter(np.float32(0.5), np.float32(0.0))
    w = np.array([[127.0, below, -below, np.nextafter(np.float32(1.5), np.float32(0))]], np.float32)
    q, _ = quantize_rows_int8(w)
    assert q[0].tolist() == [127, 0, 0, 1]


def test_round_half_away_matches_integer_cases():
    v = np.array([-3.5, -2.5, -0.5, 0.5, 2.5, 3.49, -3.51, 7.0])
    assert round_half_away(v).tolist() == [-4, -3, -1, 1, 3, 3, -4, 7]


def test_symmetric_codes_and_range():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((40, 96)) * 0.02).astype(np.float32)
    q, s = quantize_rows_int8(w)
    qn, sn = quantize_rows_int8(-w)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    assert q.dtype == np.int8 and np.abs(q.astype(int)).max() == 127 and q.min() >= -127
    # the row's largest magnitude maps to +-127, with the sign of the weight
    j = np.argmax(np.abs(w), axis=1)
    assert np.array_equal(q[np.arange(40), j].astype(int), np.where(w[np.arange(40), j] < 0, -127, 127))


def test_scale_is_row_max_over_127_and_error_within_half_step():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((16, 256)) * 0.05).astype(np.float32)
    q, s = quantize_rows_int8(w)
    assert np.array_equal(s, (np.abs(w).max(axis=1) / np.float32(127)).astype(np.float32))
    err = np.abs(w.astype(np.float64) - dequantize(q, s))
    assert np.all(err <= 0.5 * s[:, None].astype(np.float64) * (1 + 1e-6))


def test_per_channel_zero_rows_and_bf16_input():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((6, 64)) * 0.02).astype(np.float32)
    q, s = quantize_rows_int8(w)
    w2 = w.copy()
    w2[2] *= 1000.0                       # an outlier row leaves the others' codes alone
    w2[4] = 0.0
    q2, s2 = quantize_rows_int8(w2)
    for r in (0, 1, 3, 5):
        assert np.array_equal(q2[r], q[r]) and s2[r] == s[r]
    assert s2[4] == 0 and not q2[4].any()
    # bf16 storage: quantizing the bits equals quantizing their exact float values
    bits = f32_to_bf16_bits(w)
    from oracle.numerics import bf16_bits_to_f32
    qb, sb = quantize_rows_int8(bits)
    qf, sf = quantize_rows_int8(bf16_bits_to_f32(bits))
    assert np.array_equal(qb, qf) and np.array_equal(sb, sf)
