"""Attention backward: exact float64 gradients and the 8-bit emulation.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The SageAttention3 abstract (fugumt page; its title also heads an entry of
the khansong page's similar-papers list, beside the SageBwd teaser) announces
an accurate and efficient 8-bit attention for forward and backward
propagation, and gives no formats.  The readings taken here:

B1. What is differentiated: O = softmax(c Q K^T + M) V with c = sm_scale and
    M the causal mask.  Given dO, the FlashAttention backward formulas:
        D_i  = sum_c dO_ic O_ic
        dV   = P^T dO          dP = dO V^T
        dS   = P o (dP - D)     (o: elementwise; D broadcast over keys)
        dQ   = c dS K           dK = c dS^T Q
    ``exact_attention_grad`` is that, in float64 on the exact softmax.

B2. The training forward is the library's forward (INT8 Q/K codes, FP8 P~ and
    V); it also returns L_i = log2 sum_j 2^(s_ij) of its own log2-domain
    scores s (the scores of ``oracle.attention``, with K smoothing and the
    Q-smoothing bias), so that P_ij = 2^(s_ij - L_i) is its softmax.

B3. Every product of the backward takes 8-bit operands, each quantised with
    scales that are constant along that product's reduction axis:
      * S: the forward's own INT8 codes, scales and bias (P is recomputed
        exactly as the forward formed it);
      * dP = dO V^T (reduces over channels, like Q K^T): INT8 with the
        THREAD granularity's groups, dO taking the query side (one scale per
        token) and V the key side (one scale per 16-key group), no smoothing;
      * dV = P^T dO (reduces over queries, like P~ V): P to E4M3 with the
        fixed scale 1/P_r, as the forward's P~; dO to E4M3 with one scale per
        channel over all tokens, as the forward's V (without smoothing);
      * dQ = c dS K (reduces over keys): dS to E4M3 with a power-of-two scale
        per query row and 64-key group; K enters smoothed, K' = K - mean(K)
        as in the forward, to E4M3 per channel.  dS K = dS K' because every
        row of the exact dS sums to zero (the softmax does not move when all
        keys shift together), and with K' the rounding of the stored O in D
        is not multiplied by K's channel offsets;
      * dK = c dS^T Q (reduces over queries): dS to E4M3 with a power-of-two
        scale per key and 64-query group; Q to E4M3 per channel.
    The power-of-two scale of a dS group is the smallest 2^e with
    448 2^e >= the group's max |dS| (nothing saturates), the FP8 counterpart
    of the MXFP4 block exponent of the SageAttention3 FP4 reading (E8M0
    scales, e in [-127, 127]; an all-zero group has codes 0).

B4. Arithmetic: s as the forward emulation; P = fp32(2^(s - L)), 0 where
    masked (causal j > i, padded keys j >= N, padded queries i >= N);
    dP = fp32(dP_int dO_scale_i V_scale_j); D = fp32 of the float64 sum over
    the stored O and dO; t = fp32(dP - D); dS = fp32(P t); every product
    then sums the decoded codes in float64.
"""
from __future__ import annotations

import numpy as np

from .attention import LOG2E, _default_scale, emulate_block
from .fp8 import e4m3_decode, e4m3_encode
from .quant import QBLOCK, QuantParams, k_group_index, q_group_index, quant_qk, quant_v, bias_row

E4M3_MAX = 448.0
GROUP = 64              # dS scale group along a product's reduction axis
ALL_CODECS = frozenset(("s", "dp", "p", "fp8", "ds"))


# ----------------------------------------------------------------------- exact
def exact_attention_grad_head(q, k, v, do, causal=False, sm_scale=None):
    """Exact float64 (dQ, dK, dV) of one head; q, k, v, do: [N, d]."""
    q64, k64, v64, do64 = (np.asarray(x, np.float64) for x in (q, k, v, do))
    N, d = q64.shape
    c = _default_scale(d, sm_scale)
    z = (q64 @ k64.T) * c
    if causal:
        z = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, z)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    o = p @ v64
    dv = p.T @ do64
    dp = do64 @ v64.T
    dsum = (do64 * o).sum(axis=1, keepdims=True)
    ds = p * (dp - dsum)
    return c * (ds @ k64), c * (ds.T @ q64), dv


def exact_attention_grad(q, k, v, do, causal=False, sm_scale=None):
    """Exact float64 gradients over [B,H,N,d] inputs."""
    B, H = q.shape[:2]
    out = [np.empty(q.shape, np.float64) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            g = exact_attention_grad_head(q[b, h], k[b, h], v[b, h], do[b, h], causal, sm_scale)
            for o, x in zip(out, g):
                o[b, h] = x
    return tuple(out)


# ------------------------------------------------------------ 8-bit pieces
def e8m0_exponent(amax):
    """Smallest e with 448 * 2^e >= amax (float32 amax >= 0), in [-127, 127].

    For a normal amax = (1 + M / 2^23) 2^E: 448 2^(E-8) = 1.75 2^E covers it
    exactly when M <= 0.75 * 2^23, otherwise e = E - 7.  Zero or subnormal
    amax gives -127."""
    a = np.asarray(amax, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.int64)
    ef = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    e = np.where(m <= 3 * (1 << 21), ef - 127 - 8, ef - 127 - 7)
    e = np.where(ef == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def mx8_values(x, axis: int):
    """E4M3 with a power-of-two scale per GROUP consecutive elements along
    ``axis`` (float32 x, length a multiple of GROUP).  Returns the decoded
    values (float64) and the exponents (the other axes first, then the group
    index along ``axis``)."""
    x = np.asarray(x, np.float32)
    xm = np.moveaxis(x, axis, -1)
    *lead, n = xm.shape
    g = xm.reshape(*lead, n // GROUP, GROUP)
    e = e8m0_exponent(np.abs(g).max(axis=-1))
    scaled = (g.astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None]).astype(np.float32)
    vals = e4m3_decode(e4m3_encode(scaled)) * np.exp2(e.astype(np.float64))[..., None]
    return np.moveaxis(vals.reshape(*lead, n), -1, axis), e


def lse_block(qk: dict, vq: dict, b: int, h: int, qb: int, causal: bool, sm_scale=None, p_range: float = 448.0,
              quantized: bool = True):
    """L = log2 sum_j 2^(s_j) of the forward emulation's scores for the rows of
    query block qb (float32; its m and l at the end of the key loop)."""
    tr = []
    emulate_block(qk, vq, b, h, qb, causal, sm_scale, p_range, quantized=quantized, trace=tr)
    last = tr[-1]
    pscale = float(np.float32(p_range)) if quantized else 1.0
    with np.errstate(divide="ignore"):
        return (last["m"] + np.log2(last["l"] / pscale)).astype(np.float32)


def forward_with_lse(q, k, v, causal: bool, dtype: str, p: QuantParams = QuantParams(), sm_scale=None,
                     quantized=True):
    """The emulated training forward: O rounded to the I/O dtype (float32
    [B,H,N,d]), L (float32 [B,H,n_pad]) and the quantised buffers (qk, vq)."""
    from .attention import round_output
    qk, vq = quant_qk(q, k, p), quant_v(v, p)
    B, H, n_pad = qk["q_codes"].shape[:3]
    N = q.shape[2]
    o = np.full(q.shape, np.nan)
    lse = np.full((B, H, n_pad), np.nan, np.float32)
    pscale = float(np.float32(p.p_range)) if quantized else 1.0
    for b in range(B):
        for h in range(H):
            for qb in range(n_pad // QBLOCK):
                tr = []
                ob_, rows = emulate_block(qk, vq, b, h, qb, causal, sm_scale, p.p_range, quantized=quantized,
                                          trace=tr)
                o[b, h, rows] = ob_
                with np.errstate(divide="ignore"):
                    lse[b, h, qb * QBLOCK:(qb + 1) * QBLOCK] = (tr[-1]["m"] + np.log2(tr[-1]["l"] / pscale))
    return round_output(o[:, :, :N], dtype), lse, qk, vq


def prepare(q, k, v, do, o, lse, qk: dict, causal: bool, sm_scale=None, p_range: float = 448.0, codecs=None):
    """Everything the backward blocks need: the per-tensor quantisations of B3
    and D.  o and do are the stored (I/O dtype) values; lse comes from the
    forward (float32 [B,H,n_pad])."""
    codecs = ALL_CODECS if codecs is None else frozenset(codecs)
    B, H, N, d = q.shape
    n_pad = qk["n_pad"]
    pi = QuantParams(qk_bits=8, gran="thread", smooth_q=False, smooth_k=False)
    dov = quant_qk(do, v, pi, with_bias=False)            # dO on the query side, V on the key side
    pc = QuantParams(smooth_v=False, v_range=E4M3_MAX)
    fp8 = {name: quant_v(x, pc) for name, x in (("do", do), ("q", q))}
    fp8["k"] = quant_v(k, QuantParams(smooth_v=True, v_range=E4M3_MAX))     # K' = K - mean(K)
    pad = lambda x: np.concatenate([np.asarray(x, np.float64), np.zeros((B, H, n_pad - N, d))], axis=2)
    dsum = (pad(do) * pad(o)).sum(axis=-1).astype(np.float32)
    return dict(q=pad(q), k=fp8["k"]["v_smoothed"].astype(np.float64), v=pad(v), do=pad(do), qk=qk, dov=dov,
                fp8=fp8, D=dsum,
                lse=np.asarray(lse, np.float32), N=N, n_pad=n_pad, d=d, causal=causal,
                c=_default_scale(d, sm_scale), scale=_default_scale(d, sm_scale) * LOG2E,
                p_range=float(np.float32(p_range)), codecs=codecs)


def _scores(ctx, b, h, rows, cols):
    """fp32 log2-domain scores s of the forward for query rows x key cols."""
    qk, n_pad = ctx["qk"], ctx["n_pad"]
    if "s" in ctx["codecs"]:
        qmat = qk["q_codes"][b, h, rows].astype(np.float64)
        kmat = qk["k_codes"][b, h, cols].astype(np.float64)
        dq = qk["q_scale"][b, h][q_group_index(n_pad, qk["gran"])[rows]].astype(np.float64)
        dk = qk["k_scale"][b, h][k_group_index(n_pad, qk["gran"])[cols]].astype(np.float64)
        sc = dq[:, None] * dk[None, :]
    else:
        qmat = qk["q_smoothed"][b, h, rows].astype(np.float64)
        kmat = qk["k_smoothed"][b, h, cols].astype(np.float64)
        sc = 1.0
    qb = int(rows[0]) // QBLOCK
    assert np.all(rows // QBLOCK == qb), "rows of one query block"
    bias = (qk["bias"][b, h, qb] if qk.get("bias") is not None else bias_row(qk, b, h, qb)).astype(np.float64)
    return (((qmat @ kmat.T) * sc + bias[None, cols]) * ctx["scale"]).astype(np.float32)


def _tile(ctx, b, h, rows, cols):
    """P, dS (fp32) of query rows x key cols, masked entries 0."""
    N = ctx["N"]
    s = _scores(ctx, b, h, rows, cols)
    valid = (rows[:, None] < N) & (cols[None, :] < N)
    if ctx["causal"]:
        valid &= cols[None, :] <= rows[:, None]
    L = ctx["lse"][b, h, rows].astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        P = np.where(valid, np.exp2(s.astype(np.float64) - L[:, None]), 0.0).astype(np.float32)
    dov = ctx["dov"]
    if "dp" in ctx["codecs"]:
        n_pad = ctx["n_pad"]
        dpi = dov["q_codes"][b, h, rows].astype(np.float64) @ dov["k_codes"][b, h, cols].astype(np.float64).T
        sdo = dov["q_scale"][b, h][q_group_index(n_pad, "thread")[rows]].astype(np.float64)
        sv = dov["k_scale"][b, h][k_group_index(n_pad, "thread")[cols]].astype(np.float64)
        dP = (dpi * (sdo[:, None] * sv[None, :])).astype(np.float32)
    else:
        dP = (ctx["do"][b, h, rows] @ ctx["v"][b, h, cols].T).astype(np.float32)
    t = (dP.astype(np.float64) - ctx["D"][b, h, rows].astype(np.float64)[:, None]).astype(np.float32)
    dS = np.where(valid, P.astype(np.float64) * t.astype(np.float64), 0.0).astype(np.float32)
    return P, dS


def _fp8_rows(ctx, name, b, h, idx):
    """Rows idx of the per-channel E4M3 operand (decoded codes and the scale
    per channel), or the exact values with unit scales."""
    if "fp8" in ctx["codecs"]:
        f = ctx["fp8"][name]
        return e4m3_decode(f["v_codes"][b, h, idx]), f["v_scale"][b, h].astype(np.float64)
    return ctx[name][b, h, idx], np.ones(ctx["d"])


def dq_block(ctx, b, h, qb):
    """dQ rows of query block qb (float64 [128, d]); keys in 128-key tiles in
    ascending order, up to the diagonal when causal."""
    rows = qb * QBLOCK + np.arange(QBLOCK)
    key_end = min(ctx["n_pad"], (qb + 1) * QBLOCK) if ctx["causal"] else ctx["n_pad"]
    acc = np.zeros((QBLOCK, ctx["d"]))
    for k0 in range(0, key_end, QBLOCK):
        cols = k0 + np.arange(QBLOCK)
        _, dS = _tile(ctx, b, h, rows, cols)
        w = mx8_values(dS, axis=1)[0] if "ds" in ctx["codecs"] else dS.astype(np.float64)
        kv, _ = _fp8_rows(ctx, "k", b, h, cols)
        acc += w @ kv
    _, ks = _fp8_rows(ctx, "k", b, h, rows)
    return ctx["c"] * acc * ks[None, :]


def dkdv_block(ctx, b, h, kb):
    """(dK, dV) rows of key block kb (float64 [128, d] each); queries in
    128-query tiles in ascending order, from the diagonal on when causal."""
    cols = kb * QBLOCK + np.arange(QBLOCK)
    q_start = kb * QBLOCK if ctx["causal"] else 0
    dk = np.zeros((QBLOCK, ctx["d"]))
    dv = np.zeros((QBLOCK, ctx["d"]))
    for q0 in range(q_start, ctx["n_pad"], QBLOCK):
        rows = q0 + np.arange(QBLOCK)
        P, dS = _tile(ctx, b, h, rows, cols)
        if "p" in ctx["codecs"]:
            pw = e4m3_decode(e4m3_encode((P * np.float32(ctx["p_range"])).astype(np.float32))) / ctx["p_range"]
        else:
            pw = P.astype(np.float64)
        w = mx8_values(dS, axis=0)[0] if "ds" in ctx["codecs"] else dS.astype(np.float64)
        dov, _ = _fp8_rows(ctx, "do", b, h, rows)
        qv, _ = _fp8_rows(ctx, "q", b, h, rows)
        dv += pw.T @ dov
        dk += w.T @ qv
    _, dos = _fp8_rows(ctx, "do", b, h, cols)
    _, qs = _fp8_rows(ctx, "q", b, h, cols)
    return ctx["c"] * dk * qs[None, :], dv * dos[None, :]


def emulate_backward(ctx):
    """(dQ, dK, dV) float64 [B,H,N,d] of the 8-bit backward of B3/B4."""
    B, H, n_pad = ctx["q"].shape[:3]
    N, d = ctx["N"], ctx["d"]
    dq, dk, dv = (np.empty((B, H, n_pad, d)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            for blk in range(n_pad // QBLOCK):
                sl = slice(blk * QBLOCK, (blk + 1) * QBLOCK)
                dq[b, h, sl] = dq_block(ctx, b, h, blk)
                dk[b, h, sl], dv[b, h, sl] = dkdv_block(ctx, b, h, blk)
    return dq[:, :, :N], dk[:, :, :N], dv[:, :, :N]
