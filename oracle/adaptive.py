"""Adaptive choice between INT4-range and INT8 Q/K codes (TEST INFRASTRUCTURE ONLY).

The SageAttention2 abstract measures how accurate the quantized attention is
across layers and timesteps and then picks the QK precision per layer and
timestep from that measurement ("adaptive quantization").  The pages give no
formula for the measurement; the reading here, per call:

  * sample one 128-query block `q_block` of every (batch, head);
  * run the method on those rows twice, with INT4-range and with INT8 Q/K
    codes (everything else as set: granularity, smoothing, FP8 P~V), and round
    each output to the I/O type (the output the caller would receive);
  * compare both with exact attention of the same rows, over all sampled rows
    of all heads together, by cosine similarity and relative L1 distance (the
    metrics of the SageAttention2++ summary, "A.2 Datasets and Metrics");
  * choose INT4-range when its cosine similarity reaches `cos_min`, else INT8.

Built only from the pinned parts of the oracle: the quantisers, the tiled
emulation, exact attention and the metrics.
"""
from __future__ import annotations

import numpy as np

from .attention import emulate_block, exact_attention_rows, round16
from .metrics import cosine, rel_l1
from .quant import QuantParams, quant_qk, quant_v, QBLOCK


def probe_rows(N: int, q_block: int) -> np.ndarray:
    """Query rows of the sampled block that exist (the block may be ragged)."""
    r0 = QBLOCK * q_block
    if not 0 <= r0 < N:
        raise ValueError("q_block outside the sequence")
    return np.arange(r0, min(N, r0 + QBLOCK))


def probe_outputs(q, k, v, io_dtype: str, causal: bool, q_block: int, qk_bits: int, gran: str = "thread",
                  qk_format: str = "int", **kw) -> np.ndarray:
    """The method's output (rounded to io_dtype) on the sampled rows of every
    head: float64 [B, H, rows, d]."""
    B, H, N, d = q.shape
    p = QuantParams(qk_bits=qk_bits, gran=gran, qk_format=qk_format, **kw)
    qk, vq = quant_qk(q, k, p), quant_v(v, p)
    rows = probe_rows(N, q_block)
    out = np.empty((B, H, len(rows), d))
    for b in range(B):
        for h in range(H):
            o, got = emulate_block(qk, vq, b, h, q_block, causal, p_range=p.p_range)
            assert np.array_equal(got, rows)
            out[b, h] = round16(o, io_dtype)
    return out


def exact_rows(q, k, v, causal: bool, q_block: int) -> np.ndarray:
    """Exact fp64 attention on the sampled rows of every head: [B, H, rows, d]."""
    B, H, N, d = q.shape
    rows = probe_rows(N, q_block)
    out = np.empty((B, H, len(rows), d))
    for b in range(B):
        for h in range(H):
            out[b, h] = exact_attention_rows(q[b, h], k[b, h], v[b, h], rows, causal)
    return out


def probe_qk_bits(q, k, v, io_dtype: str, causal: bool, q_block: int, cos_min: float, gran: str = "thread",
                  qk4_format: str = "int", **kw) -> dict:
    """Measure INT4-range and INT8 against exact attention on the sampled rows
    and choose.  Returns cos / rel_l1 for both and qk_bits."""
    ref = exact_rows(q, k, v, causal, q_block)
    res = {}
    for bits, fmt in ((4, qk4_format), (8, "int")):
        o = probe_outputs(q, k, v, io_dtype, causal, q_block, bits, gran, fmt, **kw)
        res[f"cos_int{bits}"] = cosine(ref, o)
        res[f"rel_l1_int{bits}"] = rel_l1(ref, o)
    res["qk_bits"] = 4 if res["cos_int4"] >= cos_min else 8
    return res
