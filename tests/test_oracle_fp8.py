"""Pins for oracle.fp8 (E4M3 codes and per-head scales).

  * decoded values of landmark codes from the format's definition (zero,
    smallest subnormal, largest subnormal, smallest normal, one, 448, NaN);
  * every finite code round-trips through encode;
  * torch's CPU float8_e4m3fn conversion (a library routine) gives the same
    codes for random values and for every midpoint between neighbouring codes
    inside the finite range (the tie rule);
  * saturation and NaN handling;
  * the array form equals the scalar definition;
  * error bound: a normal-range quotient is within 2^-4 relative of its code;
  * per-head scales (scales other than 1): a value stored under scale s and
    read back is within 2^-4 relative of itself; the code is the library's
    conversion of the fp32 quotient x / s; saturation reads back as exactly
    +-448 s.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8 as F8


def test_landmark_codes():
    assert F8.decode(0x00) == 0.0
    assert F8.decode(0x01) == 2.0 ** -9
    assert F8.decode(0x07) == 7 * 2.0 ** -9
    assert F8.decode(0x08) == 2.0 ** -6
    assert F8.decode(0x38) == 1.0
    assert F8.decode(0x7E) == 448.0
    assert F8.decode(0xB8) == -1.0
    assert math.isnan(F8.decode(0x7F)) and math.isnan(F8.decode(0xFF))
    assert math.copysign(1.0, F8.decode(0x80)) < 0
    pos = F8.TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0) and len(pos) == 127


def test_finite_codes_round_trip():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert F8.encode(F8.decode(c)) == c, hex(c)


def _torch_codes(y):
    t = torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_matches_library_conversion_including_ties():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.normal(0, 30, 20000), rng.uniform(-448, 448, 20000),
                        rng.normal(0, 0.01, 5000)]).astype(np.float32)
    pos = F8.TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)      # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    y = np.concatenate([y, mids, -mids])
    assert np.array_equal(F8.quantize(y, 1.0), _torch_codes(y))


def test_saturation_and_nan():
    assert F8.encode(449.0) == 0x7E and F8.encode(1e30) == 0x7E
    assert F8.encode(-math.inf) == 0xFE and F8.encode(math.inf) == 0x7E
    assert F8.encode(464.0) == 0x7E                 # midpoint to the next exponent step
    assert F8.encode(math.nan) == 0x7F
    assert F8.encode(-0.0) == 0x80 and F8.encode(0.0) == 0x00
    assert F8.encode(2.0 ** -11) == 0x00            # below half the smallest subnormal
    assert F8.encode(-(2.0 ** -10)) == 0x80         # tie between -0 and -2^-9: even code 0


def test_array_form_equals_scalar_definition():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 3, 5000), [0.0, -0.0, np.nan, np.inf, -np.inf, 500.0,
                                                  -460.0, 1e-9]]).astype(np.float32)
    for scale in (1.0, 0.0107, 3.5):
        codes = F8.quantize(x, scale)
        y = x / np.float32(scale)
        assert [F8.encode(float(v)) for v in y] == codes.tolist()


def test_relative_error_bound_in_normal_range():
    rng = np.random.default_rng(2)
    y = rng.uniform(2.0 ** -6, 448, 20000).astype(np.float32) * rng.choice([-1, 1], 20000)
    back = F8.dequantize(F8.quantize(y, 1.0), 1.0)
    assert np.all(np.abs(back - y) <= 2.0 ** -4 * np.abs(y))


SCALES = (0.0107, 3.0 / 448, 0.37, 2.5)


def _quotients_in_normal_range(rng, n):
    """Target quotients x/s spread over E4M3's normal range, both signs."""
    mag = np.exp(rng.uniform(np.log(2.0 ** -6 * 1.01), np.log(440.0), n))
    return mag * rng.choice([-1.0, 1.0], n)


def test_scaled_round_trip_within_bound():
    """A value stored under scale s and read back is the value within the
    format's half-step: |dequantize(quantize(x, s), s) - x| <= 2^-4 |x| (plus
    the fp32 rounding of the quotient) wherever x / s is a normal E4M3
    magnitude.  Any scale misuse (ignored, inverted, applied twice) is off by
    a factor s or s^2."""
    rng = np.random.default_rng(3)
    for s in SCALES:
        x = (_quotients_in_normal_range(rng, 20000) * s).astype(np.float32)
        back = F8.dequantize(F8.quantize(x, s), s)
        xd = x.astype(np.float64)
        assert np.all(np.abs(back - xd) <= (2.0 ** -4 + 2.0 ** -22) * np.abs(xd)), s


def test_scaled_codes_equal_library_conversion_of_the_quotient():
    """The stored code is torch's float8_e4m3fn conversion of the fp32 quotient
    x / s (a library routine for the rounding, with the division done in fp32)."""
    rng = np.random.default_rng(4)
    for s in SCALES:
        x = (rng.normal(0, 150, 20000) * s).astype(np.float32)
        q = x / np.float32(s)
        inside = np.abs(q) <= 448                 # torch saturates nothing: keep the finite range
        assert np.array_equal(F8.quantize(x[inside], s), _torch_codes(q[inside]))


def test_scaled_saturation_lands_on_448_times_scale():
    """Beyond the largest code, a stored value reads back as exactly +-448 s."""
    for s in SCALES:
        s32 = float(np.float32(s))
        big = np.array([448 * s * 1.5, -448 * s * 4, 1e30, -1e30], dtype=np.float32)
        back = F8.dequantize(F8.quantize(big, s), s)
        assert back.tolist() == [448 * s32, -448 * s32, 448 * s32, -448 * s32]
