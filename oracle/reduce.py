"""Token-axis sums and means with one fixed fp32 rounding order.

The means that smooth K, Q and V (SageAttention2 abstract: "smooth Q and V";
K smoothing comes from SageAttention's precision-enhancing methods named in the
same abstract) decide integer and FP8 codes, so both sides must round them the
same way.  The pages do not fix an order; the reading used here is a pairwise
tree in token order, evaluated in fp32:

    pad the n values with +0.0 up to P = 128 * 2^ceil(log2(ceil(n / 128)))
    repeat  s[i] = s[2i] + s[2i+1]  until one value remains.

The mean is that sum divided by n (one correctly rounded fp32 division).  For a
Q block the set is the block's 128 positions, so P = 128.
"""
import math

import numpy as np


def pad_length(n: int) -> int:
    """Length the tree is padded to for n values (n >= 1)."""
    if n < 1:
        raise ValueError("empty token set")
    blocks = -(-n // 128)
    return 128 * (1 << max(0, math.ceil(math.log2(blocks))))


def canonical_sum(x, axis=-2, length=None):
    """fp32 pairwise-tree sum along ``axis`` (token order), zero padded.

    ``length`` forces the padded length (must be a power of two times 128 or
    exactly 128); by default ``pad_length(x.shape[axis])``.
    """
    s = np.moveaxis(np.asarray(x, dtype=np.float32), axis, 0)
    n = s.shape[0]
    P = pad_length(n) if length is None else length
    if P < n or (P & (P - 1)) != 0:
        raise ValueError("bad padded length")
    if P > n:
        s = np.concatenate([s, np.zeros((P - n,) + s.shape[1:], np.float32)], axis=0)
    while s.shape[0] > 1:
        s = s[0::2] + s[1::2]          # float32 + float32 -> float32, round to nearest even
    return s[0]


def canonical_mean(x, axis=-2, n=None, length=None):
    """canonical_sum / n in fp32 (n defaults to the axis length)."""
    n = np.asarray(x).shape[axis] if n is None else n
    return (canonical_sum(x, axis, length) / np.asarray(n, dtype=np.float32)).astype(np.float32)
