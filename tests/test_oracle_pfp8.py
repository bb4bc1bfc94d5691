"""Pins of the FP8 P~ step of the tiled emulation (the quantised branch).

The SageAttention2 abstract puts P~ in FP8, and the SageAttention2++ summary
("2.1 SageAttention2") gives it a fixed per-block scale: p^ = E4M3(P~ * P_r).
Three kinds of pins tie that step to something other than the oracle itself:

* a hand-worked tiny case (tests/golden/fp8_softmax_tiny.json): the codes,
  weights, running maxima, rescale factors and row sums of two key steps,
  including a maximum that moves in the second step, a subnormal tie and a
  flush to zero, and the resulting outputs;
* a precision window: with the QK and V quantisers off, the only departure
  from exact attention is rounding each P~ * P_r to E4M3.  Each weight then
  moves by at most u = 2^-4 relative (normal codes) or 2^-10 / P_r absolute
  (subnormal codes), while l sums the unrounded P~, so
  |O - O_exact| <= max|V'| (u + n_keys 2^-10 / P_r) (l >= 1 since the row
  maximum contributes P~ = 1).  The error must also be large enough to show
  the rounding happened at E4M3's precision;
* planted slips, each of which must fail one of the pins above.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.attention import emulate_block
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_softmax_tiny.json")
U8 = 2.0 ** -4       # unit roundoff of E4M3 (3 mantissa bits)


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def _run_golden(g, block=emulate_block):
    s = g["setup"]
    q, k, v = (np.array(s[n], np.float32)[None, None] for n in ("q", "k", "v"))
    p = QuantParams(smooth_q=s["smooth_q"], smooth_k=s["smooth_k"], smooth_v=s["smooth_v"], p_range=s["p_range"])
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    tr = []
    o, rows = block(qk, vq, 0, 0, 0, s["causal"], sm_scale=math.log(2.0), p_range=s["p_range"],
                    bk=s["key_step"], codecs={"p"}, trace=tr)
    return o, rows, tr, v[0, 0].astype(np.float64)


def _golden_ok(block=emulate_block):
    """True when the emulation reproduces every hand-worked value."""
    g = _golden()
    o, rows, tr, v = _run_golden(g, block)
    n = g["setup"]["N"]
    if len(tr) != len(g["steps"]):
        return False
    for st, want in zip(tr, g["steps"]):
        codes = np.array([[int(c, 16) for c in row] for row in want["codes"]], np.uint8)
        if not np.array_equal(oracle.e4m3_encode(st["P"][:n].astype(np.float32)), codes):
            return False
        if not np.array_equal(st["w"][:n], np.array(want["weights"])):
            return False
        if not np.array_equal(st["w"][:n], oracle.e4m3_decode(codes)):
            return False
        if not (np.array_equal(st["m"][:n], want["m"]) and np.array_equal(st["alpha"][:n], want["alpha"])):
            return False
        if not np.allclose(st["l"][:n], want["l"], rtol=g["l_rtol"], atol=0):
            return False
    out = g["output"]
    want_o = np.array(out["acc"]) / np.array(out["l"])[:, None]
    return bool(np.allclose(o[out["rows"]], want_o, rtol=out["rtol"], atol=0))


def test_golden_tiny_fp8_softmax():
    assert _golden_ok()


def test_golden_distinguishes_a_lagged_reference():
    # With a reference maximum that lags the running maximum by up to 4, row 0
    # keeps m = 0 in the second step and its codes differ from the hand-worked ones.
    g = _golden()
    o, rows, tr, v = _run_golden(g, lambda *a, **kw: emulate_block(*a, tau=4.0, **kw))
    assert tr[1]["m"][0] == 0.0
    assert not _golden_ok(lambda *a, **kw: emulate_block(*a, tau=4.0, **kw))


def _window_error(causal, name="image_dit", N=300, p_range=448.0, block=None):
    """max |O - O_exact| / max|V'| with only the P~ codec on, and the bound's key count."""
    import oracle.attention as oa
    w = scaled(WORKLOADS[name], B=1, H=2, N=N)
    q, k, v = make_inputs(w)
    p = QuantParams(p_range=p_range)
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    ex = oracle.exact_attention(q, k, v, causal)
    em = oa.emulate_attention(qk, vq, causal, p_range=p_range, codecs={"p"})
    return float(np.abs(em - ex).max() / np.abs(vq["v_smoothed"]).max()), N


def _window(causal, p_range):
    # Floors: early causal rows attend to a few keys, so a single rounded weight
    # carries a large share of the row; non-causal rows average the error down.
    floor = U8 / 16 if causal else U8 / 64
    return floor, lambda n: U8 + n * 2.0 ** -10 / p_range + 2e-6


@pytest.mark.parametrize("name,N", [("image_dit", 300), ("llm_prefill", 300), ("target", 640)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_range", [448.0, 224.0])
def test_fp8_p_emulation_within_rounding_window(name, N, causal, p_range):
    err, n = _window_error(causal, name, N, p_range)
    floor, ceil = _window(causal, p_range)
    assert err <= ceil(n)
    assert err >= floor, "the weights were not rounded at E4M3 precision"


def _window_ok(block_src_mutation=None):
    errs = [(_window_error(c)[0], c) for c in (False, True)]
    for err, causal in errs:
        floor, ceil = _window(causal, 448.0)
        if not (floor <= err <= ceil(300)):
            return False
    return True


def _accuracy_ok():
    """The full pipeline stays near exact attention (the bound the quantised
    emulation meets on V with channel means, where smoothing leaves a small part)."""
    w = scaled(WORKLOADS["image_dit"], B=1, H=2, N=512, qk_bits=8)
    q, k, v = make_inputs(w)
    qk, vq = oracle.quant_qk(q, k, QuantParams()), oracle.quant_v(v, QuantParams())
    import oracle.attention as oa
    with np.errstate(all="ignore"):
        m = oracle.compare(oracle.exact_attention(q, k, v), oa.emulate_attention(qk, vq, False))
    return m["cos"] >= 0.999 and m["rel_l1"] <= 0.02


# Plausible slips in the FP8 P~ branch, planted into a copy of the block
# routine by source substitution.  Each must fail the golden case, the window
# or the accuracy bound.
SLIPS = {
    "P~ not rounded to FP8": ("pw = e4m3_decode(e4m3_encode(PS))", "pw = PS.astype(np.float64)"),
    "P~ scale halved": ("pscale = float(np.float32(p_range)) * 2.0 ** -tau", "pscale = float(np.float32(p_range)) * 2.0 ** -tau / 2"),
    "P~ encoded without its scale": ("pw = e4m3_decode(e4m3_encode(PS))", "pw = e4m3_decode(e4m3_encode(P)) * pscale"),
    "l summed from the FP8 P~": ("(pw.sum(axis=1) if l_fp8 else", "(pw.sum(axis=1) if True else"),
    "V scale dropped": ("o = acc * dv[None, :] / l[:, None]", "o = acc / l[:, None]"),
    "codes against the step maximum": ("m_new = np.where(ms > m + tau, ms, m)", "m_new = np.where(np.isneginf(ms), m, ms)"),
}


@pytest.mark.parametrize("name", sorted(SLIPS))
def test_planted_fp8_p_slips_are_caught(name, monkeypatch):
    import inspect
    import textwrap
    import oracle.attention as oa
    old, new = SLIPS[name]
    src = textwrap.dedent(inspect.getsource(oa.emulate_block))
    assert src.count(old) == 1, f"mutation anchor for {name!r} not found once"
    ns = dict(vars(oa))
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    monkeypatch.setattr(oa, "emulate_block", ns["emulate_block"])
    with np.errstate(all="ignore"):
        caught = not _golden_ok(ns["emulate_block"]) or not _window_ok() or not _accuracy_ok()
    assert caught, f"planted slip {name!r} went unnoticed"
