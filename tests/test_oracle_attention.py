"""Pins of the exact attention and the tiled emulation.

Exact attention: brute force, row sums, shift invariance, closed forms.
Emulation: with every quantiser switched off it must equal exact attention up
to fp32 rounding of s and P~; that pins the tile loop, the online-softmax
bookkeeping, the causal skip, the masking of padded keys and the three
smoothing add-backs (K mean, Q block mean via the bias, V mean).
"""
import math

import numpy as np
import pytest

import oracle
import oracle.quant as oq
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled


def _brute(q, k, v, causal, scale):
    N, d = q.shape
    out = np.zeros((N, v.shape[1]))
    for i in range(N):
        keys = [j for j in range(N) if not (causal and j > i)]
        s = [scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(d)) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = math.fsum(e)
        for c in range(v.shape[1]):
            out[i, c] = math.fsum(e[t] * float(v[keys[t], c]) for t in range(len(keys))) / z
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_exact_vs_brute_force(causal):
    rng = np.random.default_rng(5)
    for (N, d) in [(1, 4), (7, 8), (16, 5)]:
        q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
        got = oracle.exact_attention(q, k, v, causal)[0, 0]
        ref = _brute(q[0, 0], k[0, 0], v[0, 0], causal, 1 / math.sqrt(d))
        assert np.abs(got - ref).max() <= 1e-12


def test_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 2, 40, 16)) for _ in range(3))
    for causal in (False, True):
        ones = oracle.exact_attention(q, k, np.ones_like(v), causal)
        assert np.abs(ones - 1).max() <= 1e-12
        base = oracle.exact_attention(q, k, v, causal)
        c = rng.standard_normal(16)
        assert np.abs(oracle.exact_attention(q, k + c, v, causal) - base).max() <= 1e-10
        assert np.abs(oracle.exact_attention(q, k, v + c, causal) - (base + c)).max() <= 1e-10


def test_exact_closed_forms():
    rng = np.random.default_rng(7)
    N, d = 33, 8
    q = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), N, axis=2)      # identical keys
    o = oracle.exact_attention(q, k, v, False)
    assert np.abs(o - v.mean(axis=2, keepdims=True)).max() <= 1e-12
    oc = oracle.exact_attention(q, k, v, True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.abs(oc - prefix).max() <= 1e-12
    o1 = oracle.exact_attention(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    assert np.abs(o1 - v[:, :, :1]).max() == 0
    kr = rng.standard_normal((1, 1, N, d))
    assert np.abs(oracle.exact_attention(q, kr, v, True)[0, 0, 0] - v[0, 0, 0]).max() <= 1e-15


CASES = [("tiny", 128, False), ("tiny", 200, True), ("llm_prefill", 333, True),
         ("image_dit", 300, False), ("long_context", 260, True), ("video_dit", 390, False)]


@pytest.mark.parametrize("name,N,causal", CASES)
@pytest.mark.parametrize("gran", ["thread", "block"])
def test_emulation_without_quantisation_is_exact(name, N, causal, gran):
    w = scaled(WORKLOADS[name], B=1, H=2, N=N)
    q, k, v = make_inputs(w)
    p = QuantParams(qk_bits=w.qk_bits, gran=gran)
    qk = oracle.quant_qk(q, k, p)
    vq = oracle.quant_v(v, p)
    ex = oracle.exact_attention(q, k, v, causal)
    # The reference maximum (lagging by up to tau) and the step size only move
    # rounding points; with identity codecs every choice is exact attention.
    for bk, tau in ((128, 0.0), (64, 0.0), (64, 2.0), (128, 3.0)):
        em = oracle.emulate_attention(qk, vq, causal, quantized=False, bk=bk, tau=tau)
        assert np.abs(em - ex).max() <= 2e-6 * (np.abs(v).max() + 1)


@pytest.mark.parametrize("smooth", [(False, False, False), (True, False, True), (False, True, False)])
def test_emulation_without_quantisation_any_smoothing(smooth):
    w = scaled(WORKLOADS["llm_prefill"], B=1, H=1, N=300)
    q, k, v = make_inputs(w)
    p = QuantParams(smooth_q=smooth[0], smooth_k=smooth[1], smooth_v=smooth[2])
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    ex = oracle.exact_attention(q, k, v, True)
    em = oracle.emulate_attention(qk, vq, True, quantized=False)
    assert np.abs(em - ex).max() <= 2e-6 * (np.abs(v).max() + 1)


def test_quantized_emulation_close_to_exact_on_tiny():
    w = WORKLOADS["tiny"]
    q, k, v = make_inputs(w)
    p = QuantParams(qk_bits=8, gran="thread")
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    m = oracle.compare(oracle.exact_attention(q, k, v), oracle.emulate_attention(qk, vq, False))
    assert m["cos"] >= 0.999
    assert m["rel_l1"] <= 0.05


def test_quantized_emulation_meets_rel_l1_with_channel_means():
    # V with nonzero channel means: smoothing keeps the FP8 error on the small part.
    w = scaled(WORKLOADS["image_dit"], B=1, H=2, N=512, qk_bits=8)
    q, k, v = make_inputs(w)
    p = QuantParams(qk_bits=8)
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    m = oracle.compare(oracle.exact_attention(q, k, v), oracle.emulate_attention(qk, vq, False))
    assert m["cos"] >= 0.999 and m["rel_l1"] <= 0.02


# --------------------------------------------------------------- planted mistakes
# Each test plants a plausible mistake in the oracle (on the CPU) and checks that
# one of the pins above catches it.
def _quant_off_error(monkeypatch=None, causal=True):
    w = scaled(WORKLOADS["llm_prefill"], B=1, H=1, N=300)
    q, k, v = make_inputs(w)
    p = QuantParams()
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    ex = oracle.exact_attention(q, k, v, causal)
    em = oracle.emulate_attention(qk, vq, causal, quantized=False)
    return np.abs(em - ex).max()


def test_planted_missing_bias_is_caught(monkeypatch):
    monkeypatch.setattr(oq, "bias_row", lambda qk, b, h, qb: np.zeros(qk["n_pad"], np.float32))
    real = oq.quant_qk

    def no_bias(q, k, p=QuantParams(), with_bias=True):
        return real(q, k, p, with_bias=False)
    monkeypatch.setattr(oracle, "quant_qk", no_bias)
    import oracle.attention as oa
    monkeypatch.setattr(oa, "bias_row", oq.bias_row)
    assert _quant_off_error() > 1e-3


def test_planted_bias_sign_is_caught(monkeypatch):
    real = oq.bias_row
    import oracle.attention as oa
    monkeypatch.setattr(oa, "bias_row", lambda qk, b, h, qb: -real(qk, b, h, qb))
    real_q = oq.quant_qk

    def no_bias(q, k, p=QuantParams(), with_bias=True):
        return real_q(q, k, p, with_bias=False)
    monkeypatch.setattr(oracle, "quant_qk", no_bias)
    assert _quant_off_error() > 1e-3


def test_planted_ignored_causal_mask_is_caught(monkeypatch):
    w = scaled(WORKLOADS["tiny"], N=130)
    q, k, v = make_inputs(w)
    ex = oracle.exact_attention(q, k, v, True)
    import oracle.attention as oa
    real_block = oa.emulate_block

    def ignore_causal(qk, vq, b, h, qb, causal, *args):
        return real_block(qk, vq, b, h, qb, False, *args)
    monkeypatch.setattr(oa, "emulate_block", ignore_causal)
    qk, vq = oracle.quant_qk(q, k), oracle.quant_v(v)
    em = oa.emulate_attention(qk, vq, True, quantized=False)
    assert np.abs(em - ex).max() > 1e-3


def test_planted_wrong_k_group_map_degrades_accuracy(monkeypatch):
    w = scaled(WORKLOADS["llm_prefill"], B=1, H=2, N=512, causal=False)
    q, k, v = make_inputs(w)
    p = QuantParams()
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    ex = oracle.exact_attention(q, k, v, False)
    good = oracle.compare(ex, oracle.emulate_attention(qk, vq, False))["rmse"]
    import oracle.attention as oa
    real = oa.k_group_index
    monkeypatch.setattr(oa, "k_group_index", lambda n, g: real(n, g) ^ 1)   # swap the two halves
    bad = oracle.compare(ex, oracle.emulate_attention(qk, vq, False))["rmse"]
    assert bad > 1.5 * good


# Plausible slips in the online-softmax bookkeeping, planted into a copy of
# the oracle's block routine by source substitution; the identity-codec check
# against exact attention must catch every one.
MUTATIONS = {
    "no O rescale": ("acc = alpha[:, None] * acc + pw @ vmat[j]", "acc = acc + pw @ vmat[j]"),
    "no l rescale": ("l = alpha * l + ", "l = l + "),
    "causal off by one": ("(j[None, :] > qi[:, None])", "(j[None, :] >= qi[:, None])"),
    "padded keys kept": ("(j[None, :] >= N) |", "(j[None, :] >= n_pad) |"),
    "alpha inverted": ("np.exp2(m - np.where", "np.exp2(-m + 2 * m - 2 * m + np.where"),
    "V mean dropped": ("+ vq[\"v_mean\"][b, h].astype(np.float64)[None, :]", "+ 0.0"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_softmax_bookkeeping_slips_are_caught(name, monkeypatch):
    import inspect
    import textwrap
    import oracle.attention as oa
    old, new = MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(oa.emulate_block))
    assert src.count(old) == 1, f"mutation anchor for {name!r} not found once"
    ns = dict(vars(oa))
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    monkeypatch.setattr(oa, "emulate_block", ns["emulate_block"])
    w = scaled(WORKLOADS["image_dit"], B=1, H=1, N=300)   # V with channel means; ragged tail
    q, k, v = make_inputs(w)
    qk, vq = oracle.quant_qk(q, k), oracle.quant_v(v)
    for causal in (True, False):
        ex = oracle.exact_attention(q, k, v, causal)
        for tau in (0.0, 2.0):
            with np.errstate(all="ignore"):
                em = oa.emulate_attention(qk, vq, causal, quantized=False, tau=tau)
            if not np.abs(em - ex).max() <= 1e-3:      # NaN counts as caught
                return
    raise AssertionError(f"planted slip {name!r} went unnoticed")


# ------------------------------------------------ 16-bit P~V (first SageAttention)
# With the 16-bit P~V the only departure from exact attention, once the QK
# quantiser is switched off, is rounding each P~ to the 16-bit type: every
# weight moves by at most the unit roundoff u (2^-8 bf16, 2^-11 fp16) relative,
# while l sums the unrounded P~, so |O - O_exact| <= u max|V| (plus fp32
# rounding of s and P~).  The bound must hold, and the error must show that
# the rounding happened at the right precision (well above the next format's u).
U16 = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def _pv16_error(kind, causal, name="image_dit", N=300):
    w = scaled(WORKLOADS[name], B=1, H=2, N=N)
    q, k, v = make_inputs(w)
    p = QuantParams(pv=kind)
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    ex = oracle.exact_attention(q, k, v, causal)
    em = oracle.emulate_attention(qk, vq, causal, codecs={"p"})     # QK quantisation off, P~ rounded
    return np.abs(em - ex).max() / np.abs(v).max()


def _pv16_floor(causal):
    # Early causal rows attend to a few keys, so single weights are large and
    # the rounding error shows at a good fraction of the bound; non-causal rows
    # average it down further.
    return 1 / 16 if causal else 1 / 64


@pytest.mark.parametrize("kind", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_pv16_emulation_within_rounding_bound(kind, causal):
    err = _pv16_error(kind, causal)
    assert err <= U16[kind] * (1 + 1e-3) + 2e-6
    assert err >= U16[kind] * _pv16_floor(causal)    # the weights really were rounded, at this precision


def test_pv16_quant_v_passes_v_through():
    w = scaled(WORKLOADS["image_dit"], B=1, H=2, N=200)
    _, _, v = make_inputs(w)
    vq = oracle.quant_v(v, QuantParams(pv="bf16"))
    assert vq["v_values"].shape == (1, 2, 256, 128)
    assert np.array_equal(vq["v_values"][:, :, :200], v.astype(np.float32))
    assert not vq["v_values"][:, :, 200:].any()
    assert (vq["v_scale"] == 1).all() and not vq["v_mean"].any()


def test_round16_matches_definition():
    # bf16: keep the top 16 bits of the fp32 word, nearest with ties to even.
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5 - 2 ** -8, 3e-39], np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0], np.float64)
    got = oracle.attention.round16(x, "bf16")
    assert np.array_equal(got[:5], want[:5])
    # a subnormal: word 0x0020AAC8, low half 0xAAC8 above the tie, so the top half rounds up to 0x0021
    assert np.float32(3e-39).view(np.uint32) == 0x0020AAC8
    assert got[5] == np.array([0x00210000], np.uint32).view(np.float32)[0]
    y = np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0, 2.0 ** -24], np.float32)
    assert np.array_equal(oracle.attention.round16(y, "fp16"), [1.0, 1.0 + 2 ** -9, 65504.0, 2.0 ** -24])


PV16_MUTATIONS = {
    "P not rounded": ("pw = round16(P, vq[\"pv\"])", "pw = P.astype(np.float64)"),
    "rounded to fp16 instead": ("pw = round16(P, vq[\"pv\"])", "pw = round16(P, \"fp16\")"),
    "weights scaled like FP8 codes": ("pw = round16(P, vq[\"pv\"])", "pw = round16(P * np.float32(28.0), vq[\"pv\"])"),
}


@pytest.mark.parametrize("name", sorted(PV16_MUTATIONS))
def test_planted_pv16_slips_are_caught(name, monkeypatch):
    import inspect
    import textwrap
    import oracle.attention as oa
    old, new = PV16_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(oa.emulate_block))
    assert src.count(old) == 1, f"mutation anchor for {name!r} not found once"
    ns = dict(vars(oa))
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    monkeypatch.setattr(oa, "emulate_block", ns["emulate_block"])
    err = _pv16_error("bf16", True)
    ok = U16["bf16"] * _pv16_floor(True) <= err <= U16["bf16"] * (1 + 1e-3) + 2e-6
    assert not ok, f"planted slip {name!r} went unnoticed"
