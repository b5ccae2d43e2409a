"""Exact number formats for the NVFP4 oracle (test infrastructure only).

Formats (techwalker.com LongLive-2.0 report summary, section 一: 4-bit E2M1
values that are finer near zero and coarser for large magnitudes, an FP8 scale
per 16 values, an FP32 scale per tensor):

* E2M1 -- 1 sign bit (bit 3), 2 exponent bits (bits 2:1, bias 1), 1 mantissa
  bit (bit 0).  Exponent field 0 is subnormal (value m/2).  No Inf, no NaN.
  The pages give no bit table; this is the plainest reading of "E2M1".
* E4M3 -- the FP8 scale.  Read as OCP E4M3FN: bias 7, exponent field 0 is
  subnormal (m/8 * 2^-6), 0x7F/0xFF are NaN, largest finite 448.

Rounding helpers here are exact:

* ``round_f64_to_binary`` rounds an fp64 value that *is* the exact real
  number to a binary format of p significand bits, RNE, with subnormals.
* ``round_sum_to_binary`` rounds the exact sum of two fp64 values (which may
  not be representable in fp64) via Knuth's TwoSum error term.
* ``round_fraction_to_binary`` rounds a ``Fraction``.
"""

from fractions import Fraction
import math

import numpy as np

# --------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------


def e2m1_decode(code: int) -> float:
    """Value of a 4-bit E2M1 code (sign bit 3, exponent bits 2:1, mantissa bit 0)."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5                       # subnormal: 2^(1-bias) * m/2
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


#: magnitudes of codes 0..7, ascending
E2M1_MAGNITUDES = np.array([e2m1_decode(c) for c in range(8)], dtype=np.float64)
#: midpoints between consecutive magnitudes; a tie at midpoint k goes to the
#: even code (k+1 even  <=>  round up)
E2M1_MIDPOINTS = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0
E2M1_MAX = float(E2M1_MAGNITUDES[-1])

# --------------------------------------------------------------------------
# E4M3 (FN)
# --------------------------------------------------------------------------


def e4m3_decode(byte: int) -> float:
    """Value of an E4M3FN byte (bias 7; 0x7F and 0xFF are NaN)."""
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return sign * mag


#: all non-negative finite E4M3 values, indexed by byte 0x00..0x7E (ascending)
E4M3_GRID = np.array([e4m3_decode(b) for b in range(0x7F)], dtype=np.float64)
E4M3_MIDPOINTS = (E4M3_GRID[:-1] + E4M3_GRID[1:]) / 2.0
E4M3_MAX = float(E4M3_GRID[-1])          # 448
E4M3_TABLE = np.array([e4m3_decode(b) for b in range(256)], dtype=np.float64)

# --------------------------------------------------------------------------
# exact rounding to binary floating-point formats
# --------------------------------------------------------------------------

F32 = (24, -126)    # (significand bits, exponent of the smallest normal)
BF16 = (8, -126)


def _ulp_exponent(v: np.ndarray, p: int, emin: int) -> np.ndarray:
    """Exponent of the unit in the last place of the p-bit format at |v|."""
    _, e = np.frexp(v)                  # |v| in [2^(e-1), 2^e)
    return np.maximum(e - 1, emin) - (p - 1)


def round_f64_to_binary(v, fmt) -> np.ndarray:
    """RNE of real values ``v`` (given exactly as fp64) to a binary format.

    ``fmt`` = (p, emin).  Subnormals are handled; overflow is not (callers
    stay in range).  Exact: scaling by a power of two is exact in fp64, and
    ``np.rint`` rounds half to even.
    """
    p, emin = fmt
    v = np.asarray(v, dtype=np.float64)
    ue = _ulp_exponent(v, p, emin)
    return np.ldexp(np.rint(np.ldexp(v, -ue)), ue)


def round_sum_to_binary(a, c, fmt) -> np.ndarray:
    """RNE of the exact real sum a + c (a, c fp64) to a binary format.

    s = fl64(a + c) and e = (a + c) - s exactly (Knuth's TwoSum).  Every
    rounding boundary of the target format is an fp64 number and fl64 is
    monotone, so fl64 lands on the same side of every boundary as the exact
    sum unless s *is* a boundary (a midpoint of the target format); there the
    sign of e decides, and e == 0 is a true tie (to even).
    """
    p, emin = fmt
    a = np.asarray(a, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    s = a + c
    bb = s - a
    e = (a - (s - bb)) + (c - bb)
    ue = _ulp_exponent(s, p, emin)
    scaled = np.ldexp(s, -ue)
    fl = np.floor(scaled)
    is_mid = (scaled - fl) == 0.5
    r = np.rint(scaled)
    r = np.where(is_mid & (e > 0), fl + 1.0, r)
    r = np.where(is_mid & (e < 0), fl, r)
    return np.ldexp(r, ue)


def round_fraction_to_binary(x: Fraction, fmt) -> float:
    """RNE of an exact rational to a binary format (p, emin); returns float."""
    p, emin = fmt
    x = Fraction(x)
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) <= a < 2^(e+1); settle e so that 2^e <= a < 2^(e+1)
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    q, r = divmod(n.numerator, n.denominator)
    twice = 2 * r
    if twice > n.denominator or (twice == n.denominator and q % 2 == 1):
        q += 1
    return sign * float(q * quantum)


def f32(x) -> np.ndarray:
    """fp64 values that are exactly fp32 (asserted)."""
    x = np.asarray(x, dtype=np.float64)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x, equal_nan=True)
    return x


# --------------------------------------------------------------------------
# bf16 / fp32 bit views used by the oracle's inputs and outputs
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """fp64 values that are exactly bf16 -> uint16 bit patterns (asserted)."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    bits = v32.view(np.uint32)
    assert not np.any(bits & 0xFFFF), "value is not a bf16 number"
    return (bits >> 16).astype(np.uint16)
