"""FP8 E4M3 ("fn" variant of the OCP 8-bit floating point formats).

The SageAttention2 abstract quantizes P~ and V to FP8; the SageAttention2++
summary ("2.1 SageAttention2", "3.1 Narrowing the FP8 Quantization Range")
keeps that choice.  The E4M3 encoding used here is the OCP one: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, subnormals for exponent field 0,
no infinities, and S.1111.111 as the only NaN pattern, so the largest finite
magnitude is 1.75 * 2^8 = 448.

Encoding is written as its definition: the nearest representable value, with a
tie going to the code whose last mantissa bit is 0.  Representable magnitudes
are monotone in the 7 low code bits, so "even code" is "even significand".
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode uint8 codes to float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


# codes 0..126 hold the non-negative finite magnitudes in increasing order
_POS = e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(x):
    """Round float32 values to E4M3 codes: nearest value, ties to the even code.

    Magnitudes above 464 (the midpoint between 448 and the NaN slot) are not
    representable and raise ValueError; the method never produces them.
    """
    x32 = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x32)):
        raise ValueError("non-finite value to encode")
    ax = np.abs(x32).astype(np.float64)
    if np.any(ax > 464.0):
        raise ValueError("magnitude above the E4M3 range")
    hi = np.searchsorted(_POS, ax, side="left")      # first magnitude >= |x|
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = np.abs(_POS[hi] - ax)
    d_lo = np.abs(ax - _POS[lo])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x32)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
