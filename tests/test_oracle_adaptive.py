"""Pins of the adaptive INT4/INT8 probe of the oracle (oracle/adaptive.py) and
of the metrics it uses.

The probe is a composition of pinned parts; what is pinned here is that
composition: the sampled rows are the right ones (checked against the
whole-tensor emulation and exact attention, a separate code path), the output
is rounded to the I/O type, INT8 and INT4-range are not swapped, and the
choice follows the stated rule.  The metrics get hand-worked values.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import adaptive
from oracle.attention import round16
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled


def test_metrics_hand_examples():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    out = np.array([[4.0, 3.0], [0.0, 0.0]])
    assert oracle.cosine(ref, out) == pytest.approx(24.0 / 25.0, abs=1e-15)   # <(3,4),(4,3)> / (5 * 5)
    assert oracle.rel_l1(ref, out) == pytest.approx(2.0 / 7.0, abs=1e-15)     # (1 + 1) / (3 + 4)
    assert oracle.cosine(ref, -ref) == pytest.approx(-1.0, abs=1e-15)
    assert oracle.rel_l1(ref, ref) == 0.0


@pytest.mark.parametrize("causal,q_block", [(False, 2), (True, 1), (True, 0)])
def test_probe_rows_match_whole_tensor_functions(causal, q_block):
    w = scaled(WORKLOADS["tiny"], N=300)         # d = 64, fp16, 3 blocks, the last ragged (44 rows)
    q, k, v = make_inputs(w)
    rows = adaptive.probe_rows(w.N, q_block)
    assert rows[0] == 128 * q_block and rows[-1] == min(w.N, 128 * (q_block + 1)) - 1
    p = QuantParams(qk_bits=4)
    full = oracle.emulate_attention(oracle.quant_qk(q, k, p), oracle.quant_v(v, p), causal)
    got = adaptive.probe_outputs(q, k, v, w.dtype, causal, q_block, 4)
    np.testing.assert_array_equal(got, round16(full[:, :, rows], w.dtype))
    ex = oracle.exact_attention(q, k, v, causal)
    np.testing.assert_allclose(adaptive.exact_rows(q, k, v, causal, q_block), ex[:, :, rows], rtol=0, atol=1e-12)


def test_outputs_are_on_the_io_grid():
    w = scaled(WORKLOADS["llm_prefill"], B=1, H=2, N=256)
    q, k, v = make_inputs(w)
    o = adaptive.probe_outputs(q, k, v, "bf16", False, 1, 8)
    np.testing.assert_array_equal(round16(o, "bf16"), o)
    o16 = adaptive.probe_outputs(q, k, v, "fp16", False, 1, 8)
    np.testing.assert_array_equal(round16(o16, "fp16"), o16)
    assert not np.array_equal(o, o16)


def test_int8_is_the_more_accurate_and_the_rule_holds():
    w = scaled(WORKLOADS["target"], H=2, N=384)
    q, k, v = make_inputs(w)
    r = adaptive.probe_qk_bits(q, k, v, w.dtype, False, 1, cos_min=0.999)
    assert r["cos_int8"] > r["cos_int4"] and r["rel_l1_int8"] < r["rel_l1_int4"]
    assert r["cos_int8"] >= 0.999 > r["cos_int4"] and r["qk_bits"] == 8
    # the rule: INT4-range exactly when its cosine similarity reaches cos_min
    c4 = r["cos_int4"]
    assert adaptive.probe_qk_bits(q, k, v, w.dtype, False, 1, cos_min=c4)["qk_bits"] == 4
    assert adaptive.probe_qk_bits(q, k, v, w.dtype, False, 1, cos_min=math.nextafter(c4, 2.0))["qk_bits"] == 8


def test_int4_chosen_where_int4_is_accurate():
    """The image-DiT recipe (V with channel means, moderate K offsets) keeps
    INT4-range above 0.999, so the probe picks it there."""
    w = scaled(WORKLOADS["image_dit"], B=1, H=2, N=256)
    q, k, v = make_inputs(w)
    r = adaptive.probe_qk_bits(q, k, v, w.dtype, False, 0, cos_min=0.999)
    assert r["cos_int4"] >= 0.999 and r["qk_bits"] == 4


def test_e4m3_held_int4_probe_equals_int8_held():
    w = scaled(WORKLOADS["image_dit"], B=1, H=2, N=200)
    q, k, v = make_inputs(w)
    a = adaptive.probe_qk_bits(q, k, v, w.dtype, True, 1, 0.999, qk4_format="int")
    b = adaptive.probe_qk_bits(q, k, v, w.dtype, True, 1, 0.999, qk4_format="int_e4m3")
    assert a == b


def test_block_outside_the_sequence_is_rejected():
    with pytest.raises(ValueError):
        adaptive.probe_rows(300, 3)
