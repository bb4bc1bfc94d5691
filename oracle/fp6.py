"""FP6 E2M3 and the register-slot packing of 6-bit Q/K codes (TEST INFRASTRUCTURE ONLY).

Every integer in [-7, 7] is exact in E2M3 (the OCP microscaling FP6 element:
1 sign bit, 2 exponent bits with bias 1, 3 mantissa bits, no infinities or
NaN), so INT4-range codes can be held in it without change of value:

    code  s ee mmm   value = (-1)^s * 2^(ee - 1) * (1 + mmm / 8)   for ee > 0
                     value = (-1)^s * mmm / 8                      for ee = 0

Packing (the operand layout of a 64-deep FP6 matrix product on gfx950, read
off the hardware with an in-bounds probe): per token, each 64-channel group j
and half h form one 32-value slot; slot value i holds channel
64 j + 16 h + i (i < 16) or 64 j + 32 + 16 h + (i - 16) (i >= 16); the 32
six-bit codes of a slot are packed little-endian (value i at bits 6 i .. 6 i
+ 5) into 24 bytes.  In a token's d bytes the first 16 of those bytes sit at
byte 16 (4 j + h) and the last 8 at byte 16 (4 j + 2 + h), followed by 8
zero bytes: the same 16-byte units an INT8 or E4M3 row gives the same
channels.
"""
import numpy as np

E2M3_MAX = 7.5


def e2m3_decode(codes):
    """Decode 6-bit codes (low 6 bits of any integer array) to float64."""
    c = np.asarray(codes).astype(np.int64) & 0x3F
    sign = np.where(c & 0x20, -1.0, 1.0)
    e = (c >> 3) & 0x3
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * mag


# non-negative magnitudes of codes 0..31, increasing
_MAG = e2m3_decode(np.arange(32))


def e2m3_encode(x):
    """Round float32 values to E2M3 codes (uint8 0..63): nearest, ties to the even code, saturating at 7.5."""
    x32 = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x32)):
        raise ValueError("non-finite value to encode")
    ax = np.minimum(np.abs(x32).astype(np.float64), E2M3_MAX)
    hi = np.minimum(np.searchsorted(_MAG, ax, side="left"), 31)
    lo = np.maximum(hi - 1, 0)
    pick_hi = ((_MAG[hi] - ax) < (ax - _MAG[lo])) | (((_MAG[hi] - ax) == (ax - _MAG[lo])) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x32), code | np.uint8(0x20), code).astype(np.uint8)


def slot_channels(d: int) -> np.ndarray:
    """[d/64, 2, 32] channel of each (group j, half h, slot value i)."""
    out = np.empty((d // 64, 2, 32), np.int64)
    for j in range(d // 64):
        for h in range(2):
            for i in range(32):
                out[j, h, i] = 64 * j + 16 * h + i if i < 16 else 64 * j + 32 + 16 * h + (i - 16)
    return out


def pack_slots(codes: np.ndarray) -> np.ndarray:
    """[..., d] 6-bit codes -> [..., d] bytes in the slot layout described above."""
    c = np.asarray(codes, np.uint8) & 0x3F
    d = c.shape[-1]
    out = np.zeros(c.shape, np.uint8)
    ch = slot_channels(d)
    for j in range(d // 64):
        for h in range(2):
            vals = c[..., ch[j, h]].astype(np.uint64)                  # [..., 32]
            packed = np.zeros(c.shape[:-1] + (24,), np.uint8)
            for i in range(32):
                for b in range(6):
                    bit = 6 * i + b
                    packed[..., bit // 8] |= (((vals[..., i] >> np.uint64(b)) & np.uint64(1)).astype(np.uint8)
                                              << np.uint8(bit % 8))
            out[..., 16 * (4 * j + h): 16 * (4 * j + h) + 16] = packed[..., :16]
            out[..., 16 * (4 * j + 2 + h): 16 * (4 * j + 2 + h) + 8] = packed[..., 16:]
    return out


def unpack_slots(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_slots: [..., d] bytes -> [..., d] 6-bit codes."""
    p = np.asarray(packed, np.uint8)
    d = p.shape[-1]
    out = np.zeros(p.shape, np.uint8)
    ch = slot_channels(d)
    for j in range(d // 64):
        for h in range(2):
            slot = np.concatenate([p[..., 16 * (4 * j + h): 16 * (4 * j + h) + 16],
                                   p[..., 16 * (4 * j + 2 + h): 16 * (4 * j + 2 + h) + 8]], axis=-1)
            for i in range(32):
                v = np.zeros(p.shape[:-1], np.uint8)
                for b in range(6):
                    bit = 6 * i + b
                    v |= ((slot[..., bit // 8] >> np.uint8(bit % 8)) & np.uint8(1)) << np.uint8(b)
                out[..., ch[j, h, i]] = v
    return out
