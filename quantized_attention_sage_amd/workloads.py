"""Seeded synthetic attention inputs (Q, K, V of shape [B, H, N, d]).

This module only draws random numbers and rounds them to the storage dtype.  It
holds none of the attention or quantisation arithmetic, so both the HIP path and
the CPU oracle can consume the very same tensors.

The workload shapes stand in for the attention calls of the model families the
SageAttention2 technical report evaluates (language, image and video
generation; abstract of "SageAttention2 Technical Report", and "A.2 Datasets
and Metrics" of the SageAttention2++ summary).  No dataset item is used: every
tensor is drawn from the distributions listed in ``WORKLOADS``.

Recipe (all draws from ``numpy.random.Generator(PCG64(seed))``, in this order):
  1. Q noise, 2. K noise, 3. V noise (each [B,H,N,d], float64),
  4. K channel offsets [B,H,1,d] shared across tokens,
  5. outlier-channel picks (one integer per (b,h) when the workload has them),
  6. V channel means [B,H,1,d] (only when the workload has them).
Each tensor is rounded once, from float64, to the workload dtype (round to
nearest even) and returned as float32 arrays holding exactly those values.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "round_to_bf16", "round_to_fp16", "scaled"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp16" | "bf16"
    causal: bool
    qk_bits: int          # 8 or 4 (INT4-range codes stored in int8)
    gran: str             # "thread" | "warp" | "block"
    seed: int
    k_offset_std: float   # std of the per-channel K offset
    k_outlier_scale: float = 0.0   # >0: one channel per 100 of K (at least one) scaled by this
    v_kind: str = "normal"         # "normal" | "channel_mean" | "student_t3"
    description: str = ""

    @property
    def ops(self) -> float:
        """Attention operations: 4*B*H*N^2*d, halved when causal."""
        o = 4.0 * self.B * self.H * self.N * self.N * self.d
        return o / 2 if self.causal else o

    def positions(self) -> int:
        return self.B * self.H * self.N * self.d


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 128, 64, "fp16", False, 8, "thread", 1, 3.0,
                     description="tiny non-causal attention, INT8 QK, FP8 PV"),
    "llm_prefill": Workload("llm_prefill", 2, 32, 4096, 128, "bf16", True, 8, "thread", 2, 2.0,
                            k_outlier_scale=8.0,
                            description="LLM-prefill causal attention, INT8 QK per thread group"),
    "image_dit": Workload("image_dit", 2, 24, 4096, 128, "bf16", False, 4, "thread", 3, 4.0,
                          v_kind="channel_mean",
                          description="image-DiT non-causal attention, INT4-range QK"),
    "video_dit": Workload("video_dit", 1, 12, 32760, 128, "bf16", False, 8, "thread", 4, 3.0,
                          description="video-DiT non-causal attention, 21x30x52-token latent"),
    "long_context": Workload("long_context", 1, 32, 32768, 128, "bf16", True, 8, "thread", 5, 3.0,
                             v_kind="student_t3",
                             description="long-context causal attention, heavy-tailed V"),
    "long_context_int4": Workload("long_context_int4", 1, 32, 32768, 128, "bf16", True, 4, "thread", 5, 3.0,
                                  v_kind="student_t3",
                                  description="long-context causal attention, INT4-range QK"),
    "target": Workload("target", 1, 32, 16384, 128, "bf16", False, 8, "thread", 6, 3.0,
                       description="B=1 H=32 N=16384 d=128 non-causal attention, INT8 QK, FP8 PV"),
    "target_causal": Workload("target_causal", 1, 32, 16384, 128, "bf16", True, 8, "thread", 6, 3.0,
                              description="B=1 H=32 N=16384 d=128 causal attention, INT8 QK, FP8 PV"),
    "target_int4": Workload("target_int4", 1, 32, 16384, 128, "bf16", False, 4, "thread", 6, 3.0,
                            description="B=1 H=32 N=16384 d=128 non-causal attention with SageAttention2's "
                                        "INT4-range QK, FP8 PV"),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values once to bfloat16 (nearest, ties to even); float32 result."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    tiny = (x != 0) & (np.abs(x) < 2.0 ** -126)
    if np.any(tiny):
        raise ValueError("value in the bfloat16 subnormal range; the generator does not handle it")
    b = x.view(np.uint64)
    drop = np.uint64(45)                      # 52 - 7 mantissa bits are dropped
    lsb = (b >> drop) & np.uint64(1)
    b = (b + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + lsb) & ~((np.uint64(1) << drop) - np.uint64(1))
    y = b.view(np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("value overflows bfloat16")
    return y.astype(np.float32)


def round_to_fp16(x: np.ndarray) -> np.ndarray:
    """Round float64 values once to IEEE half (numpy rounds double->half directly)."""
    y = np.asarray(x, dtype=np.float64).astype(np.float16)
    if not np.all(np.isfinite(y)):
        raise ValueError("value overflows float16")
    return y.astype(np.float32)


def make_inputs(w: Workload):
    """Return (q, k, v) float32 arrays [B,H,N,d] holding dtype-representable values."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = (w.B, w.H, w.N, w.d)
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    if w.v_kind == "student_t3":
        v = rng.standard_t(3.0, size=shape)
    else:
        v = rng.standard_normal(shape)
    k_off = rng.normal(0.0, w.k_offset_std, size=(w.B, w.H, 1, w.d))
    k = k + k_off
    if w.k_outlier_scale > 0:
        n_out = max(1, int(round(0.01 * w.d)))
        picks = np.stack([rng.choice(w.d, size=n_out, replace=False) for _ in range(w.B * w.H)])
        picks = picks.reshape(w.B, w.H, n_out)
        for b in range(w.B):
            for h in range(w.H):
                k[b, h, :, picks[b, h]] *= w.k_outlier_scale
    if w.v_kind == "channel_mean":
        m_c = rng.standard_normal((w.B, w.H, 1, w.d))
        v = v + 0.5 + m_c
    rnd = round_to_bf16 if w.dtype == "bf16" else round_to_fp16
    return rnd(q), rnd(k), rnd(v)


def make_grad(w: Workload):
    """The output gradient dO of a backward pass on this workload: N(0, 1)
    per element from its own stream (PCG64(seed + 1000)), rounded once to the
    dtype; float32 [B,H,N,d]."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
    g = rng.standard_normal((w.B, w.H, w.N, w.d))
    return (round_to_bf16 if w.dtype == "bf16" else round_to_fp16)(g)


def describe(w: Workload) -> dict:
    return {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype,
            "causal": w.causal, "qk_bits": w.qk_bits, "granularity": w.gran,
            "seed": w.seed, "ops": w.ops, "log2N": math.log2(w.N)}
