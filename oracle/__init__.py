"""CPU oracle for SageAttention2-style quantized attention (TEST INFRASTRUCTURE ONLY).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP kernels behind
the C ABI and their Python binding) never calls it and shares no code with it.

Two parts, each citing the passage of the pages it follows:

* ``attention.exact_attention`` -- textbook softmax attention in float64 on the
  exactly promoted fp16/bf16 inputs (the full-precision output O that the
  SageAttention2++ summary, "A.2 Datasets and Metrics", compares O' against).
* ``quant`` + ``attention.emulate_attention`` -- the quantisation pipeline of the
  SageAttention2 abstract and the SageAttention2++ summary ("2.1
  SageAttention2"): Q, K smoothing and INT8 / INT4-range quantisation with
  per-group scales, P~ and V to FP8 E4M3, and the FlashAttention-style tiled
  online softmax ("2. Preliminary").  Codes, scales and means follow fp32
  arithmetic exactly; the attention output is float64 apart from the fp32
  values that decide an FP8 code.
* ``metrics`` -- cosine similarity, relative L1 and RMSE ("A.2").
* ``backward`` -- exact float64 attention gradients and the emulation of the
  8-bit backward (the SageAttention3 abstract's 8-bit attention for forward
  and backward propagation, read as in that module's docstring).
* ``adaptive`` -- the adaptive INT4/INT8 choice of the SageAttention2
  abstract, read as a probe of one sampled query block per head.
* ``fp4`` -- MXFP4 (E2M1 codes with E8M0 scales per 32 channels) for the FP4
  microscaling of the SageAttention3 abstract.
* ``fp6`` -- E2M3 and the slot packing that holds INT4-range codes for an
  FP6 matrix product.
* ``fp8`` -- the OCP E4M3 ("fn") format, decoded from its definition and
  encoded by nearest-value search with ties to the even code.

Pins (tests that tie each function to something other than itself) live in
``tests/test_oracle_*.py``.  One reading has no pin from the pages: the pages
print no worked values for the quantized output, so agreement of this
emulation with the papers' own kernels is "parity unpinned"; what is pinned is
agreement with exact attention when quantisation is switched off, the
quantiser invariants, the codec, and the reduction order.
"""
from . import fp4, fp6, fp8, reduce, quant, attention, metrics, adaptive, backward  # noqa: F401

from .fp8 import e4m3_decode, e4m3_encode  # noqa: F401
from .reduce import canonical_sum, canonical_mean, pad_length  # noqa: F401
from .quant import QuantParams, quant_qk, quant_v, q_group_index, k_group_index  # noqa: F401
from .attention import exact_attention, exact_attention_rows, emulate_attention, emulate_block  # noqa: F401
from .metrics import cosine, rel_l1, rmse, compare  # noqa: F401
