"""MXFP4: FP4 E2M1 elements in 32-element blocks with an E8M0 power-of-two scale.

The SageAttention3 abstract (on the fugumt page) runs attention on FP4
matrix cores with microscaling; the pages fix neither the element format nor
the block size or the scale format.  The plainest reading on gfx950 is the OCP
microscaling format its scaled matrix instructions take:

* E2M1 element: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, no
  infinities or NaN.  Codes 0..7 hold the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
  6 (code 1 is the subnormal 0.5); bit 3 is the sign.
* E8M0 scale: an unsigned byte e standing for 2^(e - 127).
* a block is 32 consecutive channels of one token.

Encoding is written as its definition: the nearest representable magnitude,
a tie going to the code with mantissa bit 0 (the even code), magnitudes above
6 saturating to 6, and the sign kept (so -0.0 and small negatives give code
8).  The block exponent is the smallest s with 6 * 2^s >= amax, so the
block's largest element lands in (3, 6] and nothing saturates: the
power-of-two counterpart of the delta = amax / qmax rule of the integer
quantiser.  It is computed from the fp32 bit pattern of amax, exactly.
"""
import numpy as np

E2M1_MAX = 6.0
BLOCK = 32
E8M0_BIAS = 127

# magnitudes of codes 0..7, increasing
_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """Decode 4-bit codes (any integer array, low nibble used) to float64."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * mag


def e2m1_encode(x):
    """Round float32 values to E2M1 codes (uint8 0..15): nearest, ties to even, saturating."""
    x32 = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x32)):
        raise ValueError("non-finite value to encode")
    ax = np.minimum(np.abs(x32).astype(np.float64), E2M1_MAX)
    hi = np.minimum(np.searchsorted(_MAG, ax, side="left"), 7)     # first magnitude >= |x|
    lo = np.maximum(hi - 1, 0)
    d_hi = _MAG[hi] - ax
    d_lo = ax - _MAG[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x32), code | np.uint8(0x8), code).astype(np.uint8)


def block_exponent(amax):
    """Smallest s with 6 * 2^s >= amax (amax >= 0, float32), clamped to [-127, 127].

    For a normal amax = (1 + M / 2^23) * 2^e: 6 * 2^(e-2) = 1.5 * 2^e covers it
    exactly when M <= 2^22, otherwise s = e - 1.  amax = 0 (or below the
    normal range) gives -127, the smallest E8M0 scale.
    """
    a = np.asarray(amax, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.int64)
    e = ((bits >> 23) & 0xFF) - 127
    m = bits & 0x7FFFFF
    s = np.where(m <= (1 << 22), e - 2, e - 1)
    s = np.where(((bits >> 23) & 0xFF) == 0, -127, s)
    return np.clip(s, -127, 127).astype(np.int64)


def mx_quantize_rows(xs: np.ndarray, valid: np.ndarray):
    """MXFP4 quantisation of smoothed rows xs (float32 [..., n_pad, d]).

    Returns (codes uint8 [..., n_pad, d] one code per element, scale uint8
    [..., n_pad, d / 32] E8M0 bytes).  Padded rows get code 0 and scale byte 0.
    """
    xs = np.where(valid[:, None], xs, np.float32(0)).astype(np.float32)
    *lead, n, d = xs.shape
    blocks = xs.reshape(*lead, n, d // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1).astype(np.float32)
    s = block_exponent(amax)                                    # [..., n, d/32]
    # x / 2^s is exact in float32 here (a power-of-two scaling that stays normal
    # or rounds to code 0 anyway).
    scaled = (blocks.astype(np.float64) * np.exp2(-s.astype(np.float64))[..., None]).astype(np.float32)
    codes = e2m1_encode(scaled).reshape(*lead, n, d)
    scale = (s + E8M0_BIAS).astype(np.uint8)
    codes[..., ~valid, :] = 0
    scale[..., ~valid, :] = 0
    return codes, scale


def mx_decode_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Values (float64) of MXFP4 rows: E2M1 element times 2^(scale - 127) per 32-channel block."""
    *lead, n, d = codes.shape
    v = e2m1_decode(codes).reshape(*lead, n, d // BLOCK, BLOCK)
    v = v * np.exp2(scale.astype(np.float64) - E8M0_BIAS)[..., None]
    return v.reshape(*lead, n, d)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., d] 4-bit codes -> [..., d/2] bytes, channel 2i in the low nibble of byte i."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
