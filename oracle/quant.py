"""Smoothing and quantisation of Q, K and V (emulation, exact fp32 contract).

Follows the SageAttention2 abstract (Q, K to low-bit integers with fine-grained
scales; P~ and V to FP8; smoothing of Q and V; SageAttention's K smoothing
among the "precision-enhancing methods") and the SageAttention2++ summary,
"2.1 SageAttention2" (Q and K use per-block scales, V per-channel scales).

Readings where the pages are silent:
  * K smoothing subtracts the per-channel mean over all N tokens of a head.
  * Q smoothing subtracts the per-channel mean of each 128-token block; the
    lost term comes back as the bias dS[qb, j] = mu_Q(qb) . K'_j (unquantised K').
  * Scales are symmetric: delta = amax / qmax, codes = clamp(rint(x' * (qmax /
    amax)), -qmax, qmax) with round-half-even, qmax = 127 (INT8) or 7
    (INT4-range, stored in int8).  amax = 0 gives delta = 0 and zero codes.
  * Groups ("per-block", "warp-level", "per-thread" in the pages):
      BLOCK : Q 128-token blocks, K 64-token blocks
      WARP  : Q 32-token blocks,  K 64-token blocks
      THREAD: Q one token,         K the 16 keys {32s + 8a + 4h + b : a,b in 0..3}
              for each 32-key block s and h in {0, 1}
  * V: per-channel amax over the N tokens of a head, delta_V = amax / V_r and
    codes = E4M3(V' * (V_r / amax)); V_r defaults to 448 (the E4M3 maximum).
  * Rows past N (padding up to a multiple of 128) hold code 0 and are left out
    of every mean and amax.
  * qk_format "int_e4m3" stores the INT4-range integer codes as the E4M3 byte
    of the same integer (exact for |code| <= 15; code 0 is byte 0): the same
    numbers in the operand format of an FP8 matrix product.  "int_e2m3" holds
    them as 6-bit E2M3 codes (exact for |code| <= 7) packed in the operand
    layout of an FP6 matrix product (oracle/fp6.py).
All arithmetic that feeds a code is numpy float32 (IEEE, round to nearest even,
no fused multiply-add).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .fp4 import mx_quantize_rows, mx_decode_rows, pack_nibbles
from .fp6 import e2m3_encode, pack_slots
from .fp8 import e4m3_encode
from .reduce import canonical_mean, pad_length

GRAN_BLOCK, GRAN_WARP, GRAN_THREAD = "block", "warp", "thread"
QBLOCK = 128   # Q block (smoothing unit, attention work unit)


@dataclasses.dataclass(frozen=True)
class QuantParams:
    qk_bits: int = 8
    gran: str = GRAN_THREAD
    smooth_q: bool = True
    smooth_k: bool = True
    smooth_v: bool = True
    p_range: float = 448.0
    v_range: float = 448.0
    pv: str = "fp8"          # P~V precision: "fp8" (SageAttention2), or "bf16" / "fp16" (SageAttention)
    qk_format: str = "int"   # "int" (INT8 / INT4-range, qk_bits and gran), "int_e4m3" / "int_e2m3"
                             # (INT4-range held as E4M3 bytes / packed E2M3) or "mxfp4" (SageAttention3's FP4)

    @property
    def qmax(self) -> int:
        if self.qk_bits == 8:
            return 127
        if self.qk_bits == 4:
            return 7
        raise ValueError("qk_bits must be 8 or 4")


def n_padded(N: int) -> int:
    return -(-N // QBLOCK) * QBLOCK


def q_group_index(n_pad: int, gran: str) -> np.ndarray:
    """Group id of every (padded) query token."""
    i = np.arange(n_pad)
    if gran == GRAN_BLOCK:
        return i // 128
    if gran == GRAN_WARP:
        return i // 32
    if gran == GRAN_THREAD:
        return i
    raise ValueError(gran)


def k_group_index(n_pad: int, gran: str) -> np.ndarray:
    """Group id of every (padded) key token."""
    j = np.arange(n_pad)
    if gran in (GRAN_BLOCK, GRAN_WARP):
        return j // 64
    if gran == GRAN_THREAD:
        return 2 * (j // 32) + (j % 8) // 4
    raise ValueError(gran)


def _group_amax(row_amax: np.ndarray, groups: np.ndarray) -> np.ndarray:
    """Max of row_amax [..., n_pad] over each group id (groups cover 0..G-1)."""
    order = np.argsort(groups, kind="stable")
    g_sorted = groups[order]
    starts = np.flatnonzero(np.r_[True, g_sorted[1:] != g_sorted[:-1]])
    return np.maximum.reduceat(row_amax[..., order], starts, axis=-1).astype(np.float32)


def quantize_rows(xs: np.ndarray, valid: np.ndarray, groups: np.ndarray, qmax: int):
    """Symmetric integer quantisation of smoothed rows.

    xs: float32 [..., n_pad, d] (padded rows ignored); valid: bool [n_pad];
    groups: int [n_pad].  Returns (codes int8 [..., n_pad, d], delta float32
    [..., G]).
    """
    xs = np.where(valid[:, None], xs, np.float32(0)).astype(np.float32)
    row_amax = np.abs(xs).max(axis=-1)                       # exact
    amax = _group_amax(row_amax, groups)
    qm = np.float32(qmax)
    delta = (amax / qm).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, qm / np.where(amax > 0, amax, np.float32(1)), np.float32(0)).astype(np.float32)
    inv_rows = inv[..., groups]                               # [..., n_pad]
    prod = (xs * inv_rows[..., None]).astype(np.float32)      # one fp32 multiply
    codes = np.clip(np.rint(prod), -qmax, qmax).astype(np.int8)
    codes[..., ~valid, :] = 0
    return codes, delta


def _pad_tokens(x: np.ndarray, n_pad: int) -> np.ndarray:
    N = x.shape[-2]
    if n_pad == N:
        return np.ascontiguousarray(x, dtype=np.float32)
    pad = np.zeros(x.shape[:-2] + (n_pad - N, x.shape[-1]), np.float32)
    return np.concatenate([x.astype(np.float32), pad], axis=-2)


def quant_qk(q: np.ndarray, k: np.ndarray, p: QuantParams = QuantParams(), with_bias: bool = True):
    """Smooth and quantise Q and K ([B,H,N,d] float32 holding fp16/bf16 values).

    Returns a dict with q_codes, q_scale, q_mean ([B,H,n_pad/128,d]), k_codes,
    k_scale, k_mean ([B,H,d]), k_smoothed (fp32 K', padded rows 0) and
    bias ([B,H,n_pad/128,n_pad] fp32: mu_Q(qb) . K'_j, 0 for padded keys).
    """
    B, H, N, d = q.shape
    n_pad = n_padded(N)
    valid = np.arange(n_pad) < N
    mx = p.qk_format == "mxfp4"
    if p.qk_format not in ("int", "mxfp4", "int_e4m3", "int_e2m3"):
        raise ValueError("qk_format must be int, int_e4m3, int_e2m3 or mxfp4")
    if p.qk_format in ("int_e4m3", "int_e2m3") and p.qk_bits != 4:
        raise ValueError(f"{p.qk_format} holds INT4-range codes: qk_bits must be 4")
    qmax = None if mx else p.qmax
    qp = _pad_tokens(q, n_pad)
    kp = _pad_tokens(k, n_pad)

    # K: per-channel mean over all N valid tokens (tree over pad_length(N)).
    if p.smooth_k:
        k_mean = canonical_mean(kp[..., :N, :], axis=-2, n=N, length=pad_length(N))
    else:
        k_mean = np.zeros((B, H, d), np.float32)
    ks = np.where(valid[:, None], (kp - k_mean[..., None, :]).astype(np.float32), np.float32(0))
    if mx:
        k_codes, k_scale = mx_quantize_rows(ks, valid)
    else:
        k_codes, k_scale = quantize_rows(ks, valid, k_group_index(n_pad, p.gran), qmax)

    # Q: per-channel mean of each 128-token block over its valid tokens.
    nqb = n_pad // QBLOCK
    qb_view = qp.reshape(B, H, nqb, QBLOCK, d)
    counts = np.array([min(QBLOCK, N - QBLOCK * b) for b in range(nqb)], np.float32)
    if p.smooth_q:
        q_mean = canonical_mean(qb_view, axis=-2, n=counts[:, None], length=QBLOCK)   # [B,H,nqb,d]
    else:
        q_mean = np.zeros((B, H, nqb, d), np.float32)
    qs = (qb_view - q_mean[..., None, :]).astype(np.float32).reshape(B, H, n_pad, d)
    qs = np.where(valid[:, None], qs, np.float32(0))
    if mx:
        q_codes, q_scale = mx_quantize_rows(qs, valid)
    else:
        q_codes, q_scale = quantize_rows(qs, valid, q_group_index(n_pad, p.gran), qmax)

    # Bias that restores the Q mean: dS[qb, j] = sum_c mu_Q[qb, c] * K'[j, c].
    out = dict(q_codes=q_codes, q_scale=q_scale, q_mean=q_mean.astype(np.float32),
               k_codes=k_codes, k_scale=k_scale, k_mean=k_mean.astype(np.float32),
               k_smoothed=ks, q_smoothed=qs, bias=None,
               N=N, n_pad=n_pad, gran=p.gran, qmax=qmax, qk_format=p.qk_format)
    if mx:
        # one 4-bit code per element above; the buffers hold two per byte
        out["q_values"] = mx_decode_rows(q_codes, q_scale)
        out["k_values"] = mx_decode_rows(k_codes, k_scale)
        out["q_codes"], out["k_codes"] = pack_nibbles(q_codes), pack_nibbles(k_codes)
    elif p.qk_format == "int_e4m3":
        out["q_codes"] = e4m3_encode(q_codes.astype(np.float32))
        out["k_codes"] = e4m3_encode(k_codes.astype(np.float32))
    elif p.qk_format == "int_e2m3":
        out["q_codes"] = pack_slots(e2m3_encode(q_codes.astype(np.float32)))
        out["k_codes"] = pack_slots(e2m3_encode(k_codes.astype(np.float32)))
    if with_bias:
        out["bias"] = np.stack([[np.stack([bias_row(out, b, h, qb) for qb in range(nqb)])
                                 for h in range(H)] for b in range(B)])
    return out


def bias_row(qk: dict, b: int, h: int, qb: int) -> np.ndarray:
    """dS[qb, :] = mu_Q(qb) . K'_j in float64, rounded to fp32; 0 for padded keys."""
    row = qk["k_smoothed"][b, h].astype(np.float64) @ qk["q_mean"][b, h, qb].astype(np.float64)
    row[qk["N"]:] = 0.0
    return row.astype(np.float32)


def quant_v(v: np.ndarray, p: QuantParams = QuantParams()):
    """Smooth V by its per-channel mean and encode V' to E4M3 per channel.

    Returns dict with v_codes (uint8 [B,H,n_pad,d], token-major), v_scale
    ([B,H,d] = amax / V_r), v_mean ([B,H,d]) and v_smoothed (fp32 V').

    With p.pv = "bf16" or "fp16" (the first SageAttention's 16-bit P~V, which
    the SageAttention2 abstract contrasts with its FP8 one) V is used as given:
    v_values holds it (fp32, exact, padded rows 0), v_scale is 1 and v_mean 0.
    """
    B, H, N, d = v.shape
    n_pad = n_padded(N)
    valid = np.arange(n_pad) < N
    vp = _pad_tokens(v, n_pad)
    if p.pv != "fp8":
        if p.pv not in ("bf16", "fp16"):
            raise ValueError("pv must be fp8, bf16 or fp16")
        vals = np.where(valid[:, None], vp, np.float32(0)).astype(np.float32)
        return dict(v_values=vals, v_scale=np.ones((B, H, d), np.float32), v_mean=np.zeros((B, H, d), np.float32),
                    v_smoothed=vals, N=N, n_pad=n_pad, pv=p.pv)
    if p.smooth_v:
        v_mean = canonical_mean(vp[..., :N, :], axis=-2, n=N, length=pad_length(N))
    else:
        v_mean = np.zeros((B, H, d), np.float32)
    vs = np.where(valid[:, None], (vp - v_mean[..., None, :]).astype(np.float32), np.float32(0))
    amax = np.abs(vs).max(axis=-2).astype(np.float32)                 # [B,H,d]
    vr = np.float32(p.v_range)
    v_scale = (amax / vr).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, vr / np.where(amax > 0, amax, np.float32(1)), np.float32(0)).astype(np.float32)
    prod = (vs * inv[..., None, :]).astype(np.float32)
    v_codes = e4m3_encode(prod)
    v_codes[..., ~valid, :] = 0
    return dict(v_codes=v_codes, v_scale=v_scale, v_mean=v_mean.astype(np.float32),
                v_smoothed=vs, N=N, n_pad=n_pad, pv="fp8")
