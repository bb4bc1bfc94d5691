"""Attention: exact float64 reference and the tiled quantized emulation.

exact_attention: O = softmax(sm_scale * Q K^T + M) V in float64 on the exactly
promoted inputs; M is -inf where key j > query i when causal (square,
top-left aligned).  This is the full-precision O of the SageAttention2++
summary, "A.2 Datasets and Metrics".

emulate_attention: the FlashAttention-style tiled online softmax the
SageAttention2++ summary describes in "2. Preliminary" and "2.1 SageAttention2",
on the codes produced by ``oracle.quant``:

    for each 128-query block, key steps of BK keys in ascending order
    (steps wholly above the diagonal are skipped when causal):
      s    = (S_int * dQ_i * dK_j + dS_j) * sm_scale * log2(e)   (fp64 -> fp32)
      s    = -inf for padded keys (j >= N) and, when causal, for j > i
      m'   = max(m, max_j s)                  (the running row maximum)
      alpha = 2^(m - m')                      (1 when m' = m, 0 while m = -inf)
      P~   = 2^(s - m')  in (0, 1]             (fp64 -> fp32)
      p^   = E4M3(P~ * P_r)                   (the fixed per-block scale 1/P_r)
      l    = alpha * l + sum_j P~_j * P_r     (row sum of the fp32 P~)
      acc  = alpha * acc + sum_j dec(p^_j) * dec(v^_j)
    O = acc * dV / l + mu_V, rounded once to the output dtype.

This is the textbook online softmax: the reference maximum is the running
maximum, and every P~ of a step is formed against the maximum of all scores
seen so far.  (``tau`` > 0 is an analysis option only: the reference may then
lag the running maximum by up to tau, m' = ms only if ms > m + tau, and
P~ <= 2^tau is encoded as E4M3(P~ * P_r / 2^tau).  The library does not use it.)

With MXFP4 Q and K (qk["qk_format"] = "mxfp4", the FP4 microscaling of the
SageAttention3 abstract read as OCP MXFP4, see oracle.fp4) the codes carry
their own power-of-two block scales: S is the exact dot product of the
decoded rows and dQ = dK = 1.

With the 16-bit P~V of the first SageAttention (vq["pv"] = "bf16" or "fp16",
the setting the SageAttention2 abstract starts from) the V codes are V itself,
P~ = 2^(s - m') is rounded to that type with ties to even instead of being
scaled and encoded to E4M3, and l sums the fp32 P~ as before.

``codecs`` switches the three quantisers independently (the pins use it):
"qk" (integer / MXFP4 Q and K codes with their scales; off: the smoothed fp32
Q', K' with unit scales), "p" (P~ to E4M3 or to the 16-bit type; off: the
fp32 P~ itself) and "v" (V' to E4M3 with per-channel scales; off: the
smoothed fp32 V').  With none of them the result must equal exact attention
up to fp32 rounding of s and P~.  l sums the fp32 P~ (``l_fp8=False``, the
plain FlashAttention reading); ``l_fp8=True`` sums the rounded P~ instead, an
alternative reading that is not used.  Everything except the fp32 values that
decide a code is float64.  The running maximum changes per step, so the
emulated P~ depends on BK, which must equal the kernel's key tile (128).
"""
from __future__ import annotations

import math

import numpy as np

from .fp6 import e2m3_decode, unpack_slots
from .fp8 import e4m3_decode, e4m3_encode
from .quant import QBLOCK, q_group_index, k_group_index, bias_row

LOG2E = 1.0 / math.log(2.0)
DEFAULT_BK = 128
DEFAULT_TAU = 0.0
ALL_CODECS = frozenset(("qk", "p", "v"))


def round16(x: np.ndarray, kind: str) -> np.ndarray:
    """Round float32 values to bf16 or fp16 (nearest, ties to even); float64 result."""
    x = np.ascontiguousarray(x, np.float32)
    if kind == "fp16":
        return x.astype(np.float16).astype(np.float64)
    if kind != "bf16":
        raise ValueError(kind)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _default_scale(d: int, sm_scale):
    return 1.0 / math.sqrt(d) if not sm_scale else float(sm_scale)


def exact_attention_rows(q, k, v, rows, causal=False, sm_scale=None):
    """Exact float64 attention for one head and the given query rows.

    q, k, v: [N, d] arrays; rows: 1-D int array of query indices.  Returns
    [len(rows), d] float64.
    """
    q64 = np.asarray(q, np.float64)
    k64 = np.asarray(k, np.float64)
    v64 = np.asarray(v, np.float64)
    N, d = k64.shape
    scale = _default_scale(d, sm_scale)
    rows = np.asarray(rows)
    s = (q64[rows] @ k64.T) * scale
    if causal:
        s = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, s)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v64


def exact_attention(q, k, v, causal=False, sm_scale=None, row_block=256):
    """Exact float64 attention over [B,H,N,d] inputs."""
    B, H, N, d = q.shape
    out = np.empty((B, H, N, d), np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                out[b, h, r0:r0 + len(rows)] = exact_attention_rows(q[b, h], k[b, h], v[b, h], rows, causal, sm_scale)
    return out


def emulate_block(qk: dict, vq: dict, b: int, h: int, qb: int, causal: bool, sm_scale=None,
                  p_range: float = 448.0, bk: int = DEFAULT_BK, quantized: bool = True,
                  tau: float = DEFAULT_TAU, l_fp8: bool = False, codecs=None, trace=None):
    """Emulate one 128-query block; returns (O float64 [rows, d], rows).

    ``codecs`` (a subset of {"qk", "p", "v"}) picks the quantisers that run;
    by default all of them when ``quantized`` and none otherwise.  With none
    the smoothed fp32 values stand for the codes, scales are 1 and P~ is not
    rounded, so the result must equal exact attention up to fp32 rounding of s
    and P~, which pins the tiling, the online softmax and the smoothing
    add-backs.  ``trace``, a list, receives one dict per key step with the
    step's running maximum ``m``, the fp32 ``P`` (P~ times the code scale),
    the weights ``w`` that multiply V (decoded P~ codes), ``alpha`` and ``l``.
    """
    codecs = (ALL_CODECS if quantized else frozenset()) if codecs is None else frozenset(codecs)
    if not codecs <= ALL_CODECS:
        raise ValueError(f"unknown codecs {sorted(codecs - ALL_CODECS)}")
    N, n_pad = qk["N"], qk["n_pad"]
    d = qk["k_mean"].shape[-1]
    scale = _default_scale(d, sm_scale) * LOG2E
    q0 = qb * QBLOCK
    nrows = min(QBLOCK, N - q0)
    qi = q0 + np.arange(QBLOCK)
    fmt = qk.get("qk_format", "int")
    if "qk" not in codecs:
        qmat = qk["q_smoothed"][b, h, q0:q0 + QBLOCK].astype(np.float64)
        dq = np.ones(QBLOCK)
        kmat = qk["k_smoothed"][b, h].astype(np.float64)
        dk = np.ones(n_pad)
    elif fmt == "mxfp4":
        # MXFP4 codes carry their block scales: S is the exact dot product of the decoded rows
        qmat = qk["q_values"][b, h, q0:q0 + QBLOCK]
        dq = np.ones(QBLOCK)
        kmat = qk["k_values"][b, h]
        dk = np.ones(n_pad)
    else:
        if fmt == "int_e4m3":
            # integer codes held as E4M3 bytes: decode to the same integers
            qmat = e4m3_decode(qk["q_codes"][b, h, q0:q0 + QBLOCK])
            kmat = e4m3_decode(qk["k_codes"][b, h])
        elif fmt == "int_e2m3":
            # integer codes held as packed E2M3: unpack and decode to the same integers
            qmat = e2m3_decode(unpack_slots(qk["q_codes"][b, h, q0:q0 + QBLOCK]))
            kmat = e2m3_decode(unpack_slots(qk["k_codes"][b, h]))
        else:
            qmat = qk["q_codes"][b, h, q0:q0 + QBLOCK].astype(np.float64)
            kmat = qk["k_codes"][b, h].astype(np.float64)
        dq = qk["q_scale"][b, h][q_group_index(n_pad, qk["gran"])[q0:q0 + QBLOCK]].astype(np.float64)
        dk = qk["k_scale"][b, h][k_group_index(n_pad, qk["gran"])].astype(np.float64)
    pv16 = vq.get("pv", "fp8") != "fp8"
    if pv16:
        # 16-bit P~V: V is used as given (v_values; its scale is 1 and its mean 0)
        vmat = vq["v_values"][b, h].astype(np.float64)
        dv = np.ones(d)
        pscale = 1.0
    else:
        if "v" in codecs:
            vmat = e4m3_decode(vq["v_codes"][b, h])
            dv = vq["v_scale"][b, h].astype(np.float64)
        else:
            vmat = vq["v_smoothed"][b, h].astype(np.float64)
            dv = np.ones(d)
        # the E4M3 code of P~ is E4M3(P~ * pscale): the fixed scale 1 / P_r
        pscale = float(np.float32(p_range)) * 2.0 ** -tau if "p" in codecs else 1.0
    bias = (qk["bias"][b, h, qb] if qk.get("bias") is not None else bias_row(qk, b, h, qb)).astype(np.float64)

    key_end = min(N, q0 + QBLOCK) if causal else N
    n_steps = -(-key_end // bk)
    m = np.full(QBLOCK, -np.inf)
    l = np.zeros(QBLOCK)
    acc = np.zeros((QBLOCK, d))
    for t in range(n_steps):
        j = np.arange(t * bk, min((t + 1) * bk, n_pad))
        S = qmat @ kmat[j].T                                           # exact integers when quantized
        s = ((S * (dq[:, None] * dk[None, j]) + bias[None, j]) * scale).astype(np.float32)
        mask = (j[None, :] >= N) | (causal & (j[None, :] > qi[:, None]))
        s = np.where(mask, np.float32(-np.inf), s)
        ms = s.max(axis=1).astype(np.float64)
        m_new = np.where(ms > m + tau, ms, m)
        alpha = np.where(np.isneginf(m), 0.0, np.exp2(m - np.where(np.isneginf(m_new), 0.0, m_new)))
        base = np.where(np.isneginf(m_new), 0.0, m_new)
        P = np.exp2(s.astype(np.float64) - base[:, None]).astype(np.float32)
        PS = (P * np.float32(pscale)).astype(np.float32)               # P~ times the code scale (exact when 1)
        if "p" not in codecs:
            pw = PS.astype(np.float64)
        elif pv16:
            pw = round16(P, vq["pv"])
        else:
            pw = e4m3_decode(e4m3_encode(PS))
        l = alpha * l + (pw.sum(axis=1) if l_fp8 else P.astype(np.float64).sum(axis=1) * pscale)
        acc = alpha[:, None] * acc + pw @ vmat[j]
        m = m_new
        if trace is not None:
            trace.append(dict(keys=j, m=m.copy(), P=PS.copy(), w=pw.copy(), alpha=alpha.copy(), l=l.copy()))
    o = acc * dv[None, :] / l[:, None] + vq["v_mean"][b, h].astype(np.float64)[None, :]
    return o[:nrows], qi[:nrows]


def emulate_attention(qk: dict, vq: dict, causal: bool, sm_scale=None, p_range: float = 448.0,
                      bk: int = DEFAULT_BK, quantized: bool = True, blocks=None,
                      tau: float = DEFAULT_TAU, l_fp8: bool = False, codecs=None):
    """Emulate the whole tensor (or the (b, h, qb) triples in ``blocks``).

    Returns float64 [B,H,N,d] (rows of blocks not asked for are NaN).
    """
    B, H, n_pad = qk["q_codes"].shape[:3]
    d = qk["k_mean"].shape[-1]
    N = qk["N"]
    out = np.full((B, H, N, d), np.nan)
    if blocks is None:
        blocks = [(b, h, qb) for b in range(B) for h in range(H) for qb in range(n_pad // QBLOCK)]
    for (b, h, qb) in blocks:
        o, rows = emulate_block(qk, vq, b, h, qb, causal, sm_scale, p_range, bk, quantized, tau, l_fp8, codecs)
        out[b, h, rows] = o
    return out


def round_output(o: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 outputs once to fp16/bf16 (nearest, ties to even); float32 result."""
    o = np.asarray(o, np.float64)
    if dtype == "fp16":
        return o.astype(np.float16).astype(np.float32)
    if dtype != "bf16":
        raise ValueError(dtype)
    bits = np.ascontiguousarray(o).view(np.uint64)
    keep = np.uint64(45)
    rnd = (bits >> keep) & np.uint64(1)
    bits = (bits + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + rnd) & ~((np.uint64(1) << keep) - np.uint64(1))
    return bits.view(np.float64).astype(np.float32)
