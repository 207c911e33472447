"""FP8 (E4M3, OCP "fn" variant) K/V storage with per-KV-head scales (oracle).
Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline use it.

Source: "Inside vLLM and TGI: Paging, Versioned Schedulers and Operations",
section "Launch a pinned engine from already reviewed local artifacts": an
FP8 KV cache exists, and whether it is usable depends on the device, the
backend and the scales.  The pages fix neither the format nor the scaling.
Readings used here (plainest ones):
  * the format is E4M3 without infinities (1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 is subnormal: m/8 * 2^-6; the
    all-ones code S.1111.111 is NaN; the largest finite magnitude is 448);
  * one scale per KV head for K and one for V: a stored code c of head g
    stands for value(c) * scale_g;
  * writing x: y = x / scale_g computed in fp32 (the IEEE quotient of the two
    fp32 numbers), then rounded to the nearest E4M3 value with ties to the
    even mantissa; |y| beyond 448 saturates to +-448; NaN is stored as the
    code 0x7F.
"""
from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode(code: int) -> float:
    """Value of one E4M3 code (fp64; NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# All 256 codes' values; the positive finite ones in increasing order (codes 0..0x7E).
TABLE = np.array([decode(c) for c in range(256)])
_POS = TABLE[:0x7F]


def encode(y: float) -> int:
    """Nearest E4M3 code to y (fp64 input that is already the fp32 quotient),
    ties to the even code (even mantissa), saturating at 448, NaN -> 0x7F."""
    if math.isnan(y):
        return NAN_CODE
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = min(abs(y), MAX_FINITE)
    # the positive codes 0..0x7E are increasing in value: find the neighbours
    hi = int(np.searchsorted(_POS, a, side="left"))
    if hi < len(_POS) and _POS[hi] == a:
        return sign | hi
    lo = hi - 1
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    if d_lo < d_hi:
        c = lo
    elif d_hi < d_lo:
        c = hi
    else:
        c = lo if lo % 2 == 0 else hi        # the even code has the even mantissa
    return sign | c


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes (uint8) for the elements of x stored under `scale` (both fp32):
    `encode` of each fp32 quotient, evaluated for whole arrays at once (same
    neighbour search and tie rule)."""
    y = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float64)
    nan = np.isnan(y)
    sign = np.where(np.signbit(y), 0x80, 0)
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), MAX_FINITE)
    hi = np.searchsorted(_POS, a, side="left")
    hi_c = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi_c] - a
    tie = np.where(lo % 2 == 0, lo, hi_c)
    c = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi_c, tie))
    c = np.where(_POS[hi_c] == a, hi_c, c)
    codes = (sign | c).astype(np.uint8)
    codes[nan] = NAN_CODE
    return codes


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """fp64 values value(code) * scale."""
    return TABLE[np.asarray(codes, dtype=np.int64)] * float(np.float32(scale))
