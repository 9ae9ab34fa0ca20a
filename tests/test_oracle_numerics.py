"""Pins for the oracle's number formats (CPU only).

bf16 <-> f32 is fixed by the nanoinfer page, phase 1: widening appends 16 zero
bits, narrowing rounds half to even, and the round trip is the identity over
every bf16 value. torch's own float32 -> bfloat16 conversion is the library
special case the narrowing must agree with.
"""
import numpy as np
import torch

from oracle.numerics import bf16_bits_to_f32, f32_to_bf16_bits, round_bf16, store_kv


def test_bf16_round_trip_is_identity_on_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    back = f32_to_bf16_bits(f)
    finite = ~np.isnan(f)
    assert np.array_equal(back[finite], bits[finite])
    assert np.isnan(bf16_bits_to_f32(back[~finite])).all()


def test_bf16_widen_is_a_shift():
    assert bf16_bits_to_f32(np.array([0x3F80], np.uint16))[0] == 1.0
    assert bf16_bits_to_f32(np.array([0xC000], np.uint16))[0] == -2.0
    assert np.isinf(bf16_bits_to_f32(np.array([0x7F80], np.uint16))[0])
    assert bf16_bits_to_f32(np.array([0x0001], np.uint16)).view(np.uint32)[0] == 0x00010000


def test_bf16_round_half_to_even_ties():
    cases = {0x3F808000: 0x3F80,   # tie, even below -> stay
             0x3F818000: 0x3F82,   # tie, odd below -> up
             0x3F808001: 0x3F81,   # just above the tie -> up
             0x3F807FFF: 0x3F80,   # just below -> down
             0xBF818000: 0xBF82,   # negative tie, odd -> away (even)
             0x7F7FFFFF: 0x7F80}   # largest float rounds to +inf
    src = np.array(list(cases), dtype=np.uint32).view(np.float32)
    got = f32_to_bf16_bits(src)
    assert [int(g) for g in got] == list(cases.values())


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200_000).astype(np.float32),
                        (rng.standard_normal(50_000) * 1e-38).astype(np.float32),
                        (rng.standard_normal(50_000) * 1e30).astype(np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_nan_stays_nan():
    sig_nan = np.array([0x7F800001, 0xFFC00000], dtype=np.uint32).view(np.float32)
    out = bf16_bits_to_f32(f32_to_bf16_bits(sig_nan))
    assert np.isnan(out).all()


def test_round_bf16_goes_through_float32():
    # a value just above a bf16 tie in float64 that float32 rounds onto the tie
    tie = float(np.array([0x3F818000], np.uint32).view(np.float32)[0])
    x = tie + 1e-12
    assert np.float32(x) == np.float32(tie)
    assert round_bf16(np.array([x]))[0] == float(bf16_bits_to_f32(np.array([0x3F82], np.uint16))[0])


def test_store_kv_types():
    v = np.array([1.0, -2.5, 3.14159265358979])
    assert store_kv(v, "bf16").dtype == np.uint16
    assert store_kv(v, "f32").dtype == np.float32
    assert store_kv(v, "f32")[2] == np.float32(3.14159265358979)
