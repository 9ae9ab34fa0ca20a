"""Per-output-channel symmetric int8 weight quantization (test infrastructure only).

nanoinfer page, phase 6 (INT8 per-channel, INT4 group-wise, packing): one scale
per output row rather than per tensor; symmetric, no zero point, so a quantized
weight is just q * scale; the range is [-127, 127], so a weight and its negation
get opposite codes; rounding is half away from zero, not to even; norms and
biases are never quantized. Phase 8: the stored-int8 model computes the same
function as the "simulated" one, the same integers dequantized, which is how
the oracle runs an int8 model (dequantize, then the plain forward).

Reading where the page gives no formula: scale = max_k |w[r][k]| / 127 and the
quotient w / scale, both in float32 (the weights' precision) with IEEE
rounding; the code is the float32 quotient rounded half away from zero; a row
of zeros gets scale 0 and codes 0.
"""
from __future__ import annotations

import numpy as np

from .numerics import widen


def round_half_away(v: np.ndarray) -> np.ndarray:
    """Nearest integer, ties away from zero, of each float (exact: the fraction
    |v| - trunc(|v|) of a float is itself representable)."""
    v = np.asarray(v)
    a = np.abs(v)
    t = np.trunc(a)
    mag = t + (a - t >= 0.5)
    return np.where(v < 0, -mag, mag)


def quantize_rows_int8(w: np.ndarray):
    """(codes int8 [rows][cols], scales float32 [rows]) of a stored matrix (bf16
    bits or float32), one scale per output row."""
    w32 = widen(w).astype(np.float32)          # exact for bf16 and float32 storage
    m = np.max(np.abs(w32), axis=1)
    s = (m / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    v = (w32 / safe[:, None]).astype(np.float32)
    q = np.clip(round_half_away(v), -127, 127)
    q = np.where((s > 0)[:, None], q, 0)
    return q.astype(np.int8), s


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """q * scale per row, in float64 (exact: 8-bit times 24-bit significands)."""
    return q.astype(np.float64) * np.asarray(s, dtype=np.float64)[:, None]


MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def quantized_model(host: dict):
    """The host weights of a bf16 model with every projection matrix and the
    embedding (and an untied lm_head) replaced by their int8 codes (returned
    separately) and by the dequantized float64 matrices the oracle forward uses;
    norm gains and biases unchanged. Returns (dequantized host dict, codes dict)."""
    deq = {k: v for k, v in host.items() if k != "layers"}
    codes = {}
    for k in ("embed", "lm_head"):
        if host.get(k) is not None:
            q, s = quantize_rows_int8(host[k])
            codes[k] = (q, s)
            deq[k] = dequantize(q, s)
    deq["layers"] = []
    codes["layers"] = []
    for L in host["layers"]:
        M, C = dict(L), {}
        for k in MATRICES:
            q, s = quantize_rows_int8(L[k])
            C[k] = (q, s)
            M[k] = dequantize(q, s)
        deq["layers"].append(M)
        codes["layers"].append(C)
    return deq, codes
