"""Number formats used by the oracle (test infrastructure only).

bf16 <-> f32 follows the nanoinfer page, phase 1 (safetensors reader): bf16 is
float32 with the low 16 mantissa bits removed, so widening appends 16 zero bits
(exact for every pattern, infinities and NaNs included) and narrowing rounds
half to even; the round trip is the identity on every bf16 pattern.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bit patterns (uint16) to float32 by a 16-bit left shift."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Narrow float32 to bf16 bits, round half to even; NaN stays a quiet NaN."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    high = u >> 16
    halfway = 0x8000
    round_up = (low > halfway) | ((low == halfway) & ((high & 1) == 1))
    out = (high + round_up.astype(np.uint64)) & 0xFFFF
    nan = np.isnan(f)
    out = np.where(nan, (high | 0x0040) & 0xFFFF, out)
    return out.astype(np.uint16)


def widen(a: np.ndarray) -> np.ndarray:
    """A stored tensor as float64: uint16 arrays are bf16 bits, float32 is taken as is."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    if a.dtype == np.float32 or a.dtype == np.float64:
        return a.astype(np.float64)
    raise TypeError(f"oracle: unsupported stored dtype {a.dtype}")


def round_f32(x: np.ndarray) -> np.ndarray:
    """The float32 value nearest to x (round half to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round a float64 value to float32 and then to bf16, as a kernel holding the
    value in float32 would store it; returned as float64."""
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))
                            ).astype(np.float64)


def store_kv(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Encode float64 values in the cache's storage type (bf16 bits or float32)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if kv_dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if kv_dtype == "f32":
        return x32
    raise ValueError(kv_dtype)
