"""The two small floating-point formats of NVFP4, decoded and encoded from their
definitions.  TEST INFRASTRUCTURE ONLY (see the package docstring).

NVFP4 (pages: "GLM-5.3-Flash-NVFP4-h -- W4A16 dense-side quantization",
"Config expectations": 4-bit weights, group size 16) stores

* each weight as a 4-bit E2M1 code: 1 sign bit, 2 exponent bits (bias 1),
  1 mantissa bit, no infinities and no NaN (OCP Microscaling v1.0, FP4);
* each group scale as an 8-bit E4M3 byte of the "FN" flavour: 1 sign bit,
  4 exponent bits (bias 7), 3 mantissa bits, no infinities, the two patterns
  with all exponent and mantissa bits set are NaN, largest finite value 448
  (OCP 8-bit floating point specification).

Encoding rounds to the nearest representable value, ties to the code whose
least significant bit is 0 ("round half to even" on the code), and saturates
at the largest finite magnitude instead of producing NaN.  These are readings:
the pages print neither format nor a rounding rule.

Pins (tests/test_oracle_formats.py): the E2M1 decode is checked against the
eight magnitudes written out from the format definition and against its sign
symmetry; the E4M3 decode against torch's ``float8_e4m3fn`` for all 256 bytes;
both encoders against every midpoint between neighbouring values, one fp32
ulp either side, saturation, signs, and for E4M3 against torch's own RNE
conversion on [0, 464).
"""

import numpy as np


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (0..15) as float64.

    Bit 3 is the sign, bits 2..1 the exponent field ``e``, bit 0 the mantissa
    ``m``.  ``e == 0`` encodes the subnormal ``m * 0.5``; otherwise the value is
    ``2**(e - 1) * (1 + m / 2)``.  Code 8 is negative zero.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(sign == 1, -mag, mag).astype(np.float64)


# Magnitudes of codes 0..7 in code order, built from the decoder above.
E2M1_MAGNITUDES = e2m1_decode(np.arange(8))


def e4m3_decode(b):
    """Value of each E4M3 ("FN") byte as float64; 0x7F and 0xFF decode to NaN.

    Exponent field ``e == 0`` is subnormal: ``m * 2**-9``; otherwise
    ``2**(e - 7) * (1 + m / 8)``.
    """
    b = np.asarray(b).astype(np.int64)
    sign = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def _nearest_code(x, table):
    """Index of the entry of the ascending ``table`` nearest to ``x`` (x >= 0).

    Each midpoint of two neighbouring entries is exact in float64 (both
    entries have few significant bits), so comparing the float64 image of an
    fp32 ``x`` against it decides the rounding exactly.  A tie goes to the
    even index; anything beyond the last entry saturates to it.
    """
    x = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(table, x, side="left")       # first entry >= x
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    mid = 0.5 * (table[lo] + table[hi])
    pick_hi = (x > mid) | ((x == mid) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(x >= table[-1], len(table) - 1, idx)
    return idx.astype(np.int64)


_E4M3_POSITIVE = e4m3_decode(np.arange(0x7F))   # codes 0x00..0x7E, ascending


def e4m3_encode(x):
    """E4M3 byte nearest to each non-negative finite fp32 value.

    Round to nearest, ties to the even code, saturate at 448 (0x7E).  Group
    scales are never negative, so only the non-negative half is needed; a
    negative or NaN input raises.
    """
    x = np.asarray(x, dtype=np.float32)
    if np.any(~(x >= 0)):
        raise ValueError("e4m3_encode expects non-negative, non-NaN values")
    return _nearest_code(x, _E4M3_POSITIVE).astype(np.uint8)


def e2m1_encode(q):
    """E2M1 code (0..15) nearest to each fp32 value ``q``.

    The magnitude rounds to the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties
    to the even code, saturating at 6.  The sign bit copies the sign bit of
    ``q`` (IEEE), so a negative value that rounds to zero gives code 8 (-0).
    """
    q = np.asarray(q, dtype=np.float32)
    if np.any(np.isnan(q)):
        raise ValueError("e2m1_encode got NaN")
    mag_code = _nearest_code(np.abs(q), E2M1_MAGNITUDES)
    return (mag_code | (np.signbit(q).astype(np.int64) << 3)).astype(np.uint8)
