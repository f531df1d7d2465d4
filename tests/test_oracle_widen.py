"""Pins for the oracle's bf16 -> fp64 widening, which every attention
comparison goes through (both the oracle's inputs and the kernels' bf16
outputs are widened by it).

bf16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits
(bias 127), 7 fraction bits. The widening must be exact. It is pinned
against two things other than itself:
  * torch's own bfloat16 -> float64 conversion, over every bit pattern
    that is not a NaN;
  * the IEEE definition of the format, evaluated with exact rational
    arithmetic (sign * 2^(e-127) * (1 + f/128) for normal numbers,
    sign * 2^-126 * f/128 for subnormals), plus hand-picked values.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.attention import widen_bf16

# signalling NaN patterns raise numpy's "invalid value" flag when widened
pytestmark = pytest.mark.filterwarnings("ignore:invalid value encountered in cast")

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
EXP = (ALL.astype(np.uint32) >> 7) & 0xFF
FRAC = ALL.astype(np.uint32) & 0x7F
NOT_NAN = ~((EXP == 0xFF) & (FRAC != 0))


def ieee_bf16(bits: int):
    """The value of a bf16 bit pattern from the format's definition."""
    sign = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return float("nan") if f else sign * float("inf")
    if e == 0:
        v = Fraction(f, 128) * Fraction(1, 2 ** 126)
    else:
        v = (1 + Fraction(f, 128)) * (Fraction(2) ** (e - 127))
    return float(sign * v) if v != 0 else (-0.0 if sign < 0 else 0.0)


def test_every_pattern_matches_torch():
    got = widen_bf16(ALL)
    ref = torch.from_numpy(ALL.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert got.dtype == np.float64
    np.testing.assert_array_equal(got[NOT_NAN], ref[NOT_NAN])
    # signs of zeros and infinities too
    assert np.array_equal(np.signbit(got[NOT_NAN]), np.signbit(ref[NOT_NAN]))
    assert np.all(np.isnan(got[~NOT_NAN]))


def test_every_pattern_matches_the_format_definition():
    got = widen_bf16(ALL)
    for b in range(1 << 16):
        want = ieee_bf16(b)
        if want != want:          # NaN
            assert np.isnan(got[b])
        else:
            assert got[b] == want and np.signbit(got[b]) == np.signbit(want), hex(b)


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x3F00, 0.5),
    (0x0001, 2.0 ** -133), (0x8001, -(2.0 ** -133)), (0x0080, 2.0 ** -126),
    (0x7F7F, float.fromhex("0x1.fep127")), (0x0000, 0.0), (0x8000, -0.0),
    (0x7F80, float("inf")), (0xFF80, float("-inf")),
])
def test_hand_values(bits, value):
    got = widen_bf16(np.array([bits], dtype=np.uint16))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_shape_is_kept():
    x = ALL[:24].reshape(2, 3, 4)
    assert widen_bf16(x).shape == (2, 3, 4)
