"""Pins of the oracle's reduction order, smoothing means and quantisers."""
import json
import math
import os
import sys

import numpy as np
import pytest

import oracle
import oracle.quant as oq
from oracle.fp8 import e4m3_decode
from oracle.quant import QuantParams, quantize_rows, k_group_index, q_group_index, bias_row, n_padded
from oracle.reduce import canonical_sum, canonical_mean, pad_length
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled, round_to_bf16

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _hex32(h):
    return np.array([int(h, 16)], np.uint32).view(np.float32)[0]


# ----------------------------------------------------------------- reduction order
def test_pad_length_values():
    assert [pad_length(n) for n in (1, 127, 128, 129, 256, 640, 1000, 4096, 32760, 32768)] == \
           [128, 128, 128, 256, 256, 1024, 1024, 4096, 32768, 32768]


def test_canonical_sum_hand_examples():
    g = json.load(open(os.path.join(GOLD, "canonical_sum_examples.json")))
    for ex in g["examples"]:
        vals = np.array([_hex32(h) for h in ex["values_hex"]], np.float32)
        got = canonical_sum(vals[:, None], axis=0)[0]
        assert got.view(np.uint32) == int(ex["tree_sum_hex"], 16), ex["name"]


def test_canonical_sum_error_bound_vs_fsum():
    rng = np.random.default_rng(3)
    for n in (1, 5, 128, 300, 4096, 9000):
        x = rng.standard_normal((n, 4)).astype(np.float32) * np.float32(3.0)
        got = canonical_sum(x, axis=0).astype(np.float64)
        levels = math.ceil(math.log2(pad_length(n)))
        for c in range(4):
            exact = math.fsum(x[:, c].astype(np.float64))
            bound = levels * 2.0 ** -24 * np.abs(x[:, c]).astype(np.float64).sum() * (1 + 1e-6)
            assert abs(got[c] - exact) <= bound


@pytest.mark.parametrize("n", [1, 77, 128, 1000, 8192, 32760, 32768])
def test_constant_channel_mean_is_exact_bf16(n):
    for c in (1.0, -3.140625, 0.0078125, 96.5):
        x = np.full((n, 1), c, np.float32)
        assert canonical_mean(x, axis=0, n=n, length=pad_length(n))[0] == np.float32(c)


def test_constant_channel_mean_is_exact_fp16():
    c = np.float32(np.float16(1.2509765625))     # 11 significant bits
    for n in (3, 1024, 8192):
        x = np.full((n, 1), c, np.float32)
        assert canonical_mean(x, axis=0, n=n, length=pad_length(n))[0] == c


# ----------------------------------------------------------------- integer quantiser
def test_quantiser_hand_examples():
    g = json.load(open(os.path.join(GOLD, "quant_examples.json")))
    for ex in g["examples"]:
        row = np.array(ex["row"], np.float32)[None, :]
        codes, delta = quantize_rows(row, np.array([True]), np.array([0]), ex["qmax"])
        assert codes[0].tolist() == ex["codes"]
        assert delta[0].view(np.uint32) == int(ex["scale_hex"], 16)


def test_group_maps():
    n_pad = 256
    kt = k_group_index(n_pad, "thread")
    for g in range(n_pad // 16):
        keys = np.flatnonzero(kt == g)
        s, h = divmod(g, 2)
        expect = sorted(32 * s + 8 * a + 4 * h + b for a in range(4) for b in range(4))
        assert keys.tolist() == expect
    assert np.array_equal(k_group_index(n_pad, "block"), np.arange(n_pad) // 64)
    assert np.array_equal(q_group_index(n_pad, "warp"), np.arange(n_pad) // 32)
    assert np.array_equal(q_group_index(n_pad, "block"), np.arange(n_pad) // 128)
    assert np.array_equal(q_group_index(n_pad, "thread"), np.arange(n_pad))


@pytest.mark.parametrize("gran", ["thread", "warp", "block"])
@pytest.mark.parametrize("bits", [8, 4])
def test_quantiser_invariants(gran, bits):
    w = scaled(WORKLOADS["llm_prefill"], B=1, H=2, N=333)
    q, k, _ = make_inputs(w)
    p = QuantParams(qk_bits=bits, gran=gran)
    qk = oracle.quant_qk(q, k, p, with_bias=False)
    qmax = p.qmax
    n_pad = qk["n_pad"]
    for codes, scale, xs, groups in ((qk["q_codes"], qk["q_scale"], qk["q_smoothed"], q_group_index(n_pad, gran)),
                                     (qk["k_codes"], qk["k_scale"], qk["k_smoothed"], k_group_index(n_pad, gran))):
        assert np.abs(codes.astype(int)).max() <= qmax
        assert np.all(codes[:, :, w.N:] == 0)
        d_rows = scale[..., groups].astype(np.float64)[..., None]
        err = np.abs(xs.astype(np.float64) - d_rows * codes)
        assert np.all(err <= d_rows * (0.5 + 1e-5))
        # every group with a nonzero amax reaches qmax
        for b in range(codes.shape[0]):
            for h in range(codes.shape[1]):
                rowmax = np.abs(codes[b, h].astype(int)).max(axis=1)
                gmax = np.zeros(groups.max() + 1, int)
                np.maximum.at(gmax, groups, rowmax)
                assert np.all((gmax == qmax) | (scale[b, h] == 0))


def test_k_smoothing_centres_channels_and_kills_constant_channels():
    w = scaled(WORKLOADS["tiny"], N=300)
    q, k, _ = make_inputs(w)
    k[:, :, :, 5] = np.float32(2.5)                 # a constant channel
    qk = oracle.quant_qk(q, k, QuantParams(), with_bias=False)
    ks = qk["k_smoothed"][:, :, :w.N].astype(np.float64)
    assert np.all(ks[..., 5] == 0)
    assert np.all(qk["k_mean"][..., 5] == np.float32(2.5))
    scale = np.abs(k).mean(axis=2)
    assert np.all(np.abs(ks.mean(axis=2)) <= 1e-5 * scale + 1e-7)


def test_q_block_means_use_only_valid_tokens():
    w = scaled(WORKLOADS["tiny"], N=200)            # second block has 72 valid tokens
    q, k, _ = make_inputs(w)
    qk = oracle.quant_qk(q, k, QuantParams(), with_bias=False)
    for qb, (r0, r1) in enumerate([(0, 128), (128, 200)]):
        for c in range(0, 64, 7):
            exact = math.fsum(q[0, 0, r0:r1, c].astype(np.float64)) / (r1 - r0)
            assert abs(qk["q_mean"][0, 0, qb, c] - exact) <= 8 * 2 ** -24 * np.abs(q[0, 0, r0:r1, c]).mean() + 1e-12


def test_bias_brute_force():
    w = scaled(WORKLOADS["tiny"], N=140, d=64)
    q, k, _ = make_inputs(w)
    qk = oracle.quant_qk(q, k, QuantParams())
    for (b, h, qb, j) in [(0, 0, 0, 3), (0, 1, 1, 139), (0, 1, 0, 130), (0, 0, 1, 0)]:
        mu = qk["q_mean"][b, h, qb].astype(np.float64)
        kp = (k[b, h, j].astype(np.float32) - qk["k_mean"][b, h]).astype(np.float32).astype(np.float64)
        exact = math.fsum(mu[c] * kp[c] for c in range(64))
        got = float(qk["bias"][b, h, qb, j])
        assert abs(got - exact) <= abs(exact) * 2 ** -23 + 1e-30
    assert np.all(qk["bias"][..., 140:] == 0)


# ----------------------------------------------------------------- V to FP8
@pytest.mark.parametrize("vr", [448.0, 4.5])
def test_v_quantiser(vr):
    w = scaled(WORKLOADS["image_dit"], B=1, H=2, N=257)
    _, _, v = make_inputs(w)
    vq = oracle.quant_v(v, QuantParams(v_range=vr))
    dec = e4m3_decode(vq["v_codes"])
    assert np.all(vq["v_codes"][:, :, w.N:] == 0)
    # the channel extreme lands on exactly +-V_r
    assert np.allclose(np.abs(dec[:, :, :w.N]).max(axis=2), vr)
    # E4M3 relative step: |V' - dV * dec| <= 2^-4 |V'| (normal) or half a subnormal step
    vs = vq["v_smoothed"].astype(np.float64)
    dv = vq["v_scale"].astype(np.float64)[:, :, None, :]
    err = np.abs(vs - dv * dec)
    assert np.all(err <= 2.0 ** -4 * np.abs(vs) * (1 + 1e-6) + dv * 2.0 ** -10 * (1 + 1e-6))
    mean_exact = v[:, :, :w.N].astype(np.float64).mean(axis=2)
    assert np.all(np.abs(vq["v_mean"] - mean_exact) <= 9 * 2 ** -24 * np.abs(v).mean(axis=2) + 1e-12)


def test_sa2pp_narrowed_ranges_bound_the_codes():
    # SageAttention2++ summary, 3.1: P_r = 224 and V_r = 4.5 (example bounds |p| <= 224, |v| <= 9).
    w = scaled(WORKLOADS["tiny"], N=256)
    q, k, v = make_inputs(w)
    p = QuantParams(p_range=224.0, v_range=4.5)
    vq = oracle.quant_v(v, p)
    assert np.abs(e4m3_decode(vq["v_codes"])).max() == 4.5
    qk = oracle.quant_qk(q, k, p)
    ex = oracle.exact_attention(q, k, v)
    em = oracle.emulate_attention(qk, vq, False, p_range=224.0)
    assert oracle.cosine(ex, em) >= 0.999


def test_generators_round_like_torch():
    import torch
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100_000).astype(np.float32).astype(np.float64)   # single rounding in torch too
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_generators_are_deterministic_and_padded_sizes():
    w = scaled(WORKLOADS["video_dit"], H=1, N=300)
    a = make_inputs(w)
    b = make_inputs(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert n_padded(300) == 384 and n_padded(32760) == 32768


# Plausible slips in the integer quantiser, planted into a copy of the
# oracle's routine by source substitution: the hand-worked examples or the
# invariants above must catch each one.
QUANT_MUTATIONS = {
    "floor instead of rint": ("np.rint(prod)", "np.floor(prod)"),
    "amax without abs": ("np.abs(xs).max(axis=-1)", "xs.max(axis=-1)"),
    "scale off by one": ("delta = (amax / qm)", "delta = (amax / (qm + 1))"),
    "no clamp": ("np.clip(np.rint(prod), -qmax, qmax)", "np.rint(prod * np.float32(1.0001))"),
    "row amax instead of group amax": ("inv_rows = inv[..., groups]",
                                       "inv_rows = np.where(row_amax > 0, qm / np.maximum(row_amax, 1e-30), 0)"),
}


@pytest.mark.parametrize("name", sorted(QUANT_MUTATIONS))
def test_planted_quantiser_slips_are_caught(name, monkeypatch):
    import inspect
    import textwrap
    old, new = QUANT_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(oq.quantize_rows))
    assert src.count(old) == 1, f"mutation anchor for {name!r} not found once"
    ns = dict(vars(oq))
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    monkeypatch.setattr(oq, "quantize_rows", ns["quantize_rows"])
    monkeypatch.setattr(sys.modules[__name__], "quantize_rows", ns["quantize_rows"])
    caught = 0
    for check in (test_quantiser_hand_examples, lambda: test_quantiser_invariants("thread", 8)):
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, OverflowError):
            caught += 1
    assert caught, f"planted slip {name!r} went unnoticed"


# ------------------------------------------------- INT4-range codes held as E4M3
# E4M3 bytes of the integers 0..7, written out from the format (bias 7, three
# mantissa bits): 1 = 1.0 x 2^0 -> 0 0111 000; 3 = 1.5 x 2^1 -> 0 1000 100; ...
E4M3_OF_INT = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E}


def test_int_e4m3_byte_table():
    ints = np.arange(-7, 8)
    want = np.array([E4M3_OF_INT[abs(i)] | (0x80 if i < 0 else 0) for i in ints], np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(ints.astype(np.float32)), want)
    np.testing.assert_array_equal(e4m3_decode(want), ints.astype(np.float64))


@pytest.mark.parametrize("gran", ["thread", "warp", "block"])
def test_int_e4m3_holds_the_int4_codes(gran):
    """The E4M3-held codes are the INT4-range codes byte for byte through the
    table above, with identical scales, means and bias, and the emulation of
    the two formats gives identical outputs."""
    w = scaled(WORKLOADS["image_dit"], B=1, H=2, N=300)
    q, k, v = make_inputs(w)
    pi = QuantParams(qk_bits=4, gran=gran)
    pe = QuantParams(qk_bits=4, gran=gran, qk_format="int_e4m3")
    a, b = oracle.quant_qk(q, k, pi), oracle.quant_qk(q, k, pe)
    table = np.array([E4M3_OF_INT[abs(i)] | (0x80 if i < 0 else 0) for i in range(-7, 8)], np.uint8)
    for n in ("q_codes", "k_codes"):
        assert b[n].dtype == np.uint8
        np.testing.assert_array_equal(b[n], table[a[n].astype(np.int64) + 7], err_msg=n)
    for n in ("q_scale", "k_scale", "q_mean", "k_mean", "bias"):
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
    vq = oracle.quant_v(v, pi)
    for causal in (False, True):
        np.testing.assert_array_equal(oracle.emulate_attention(a, vq, causal), oracle.emulate_attention(b, vq, causal))


def test_int_e4m3_needs_int4_range():
    q = np.zeros((1, 1, 128, 64), np.float32)
    with pytest.raises(ValueError):
        oracle.quant_qk(q, q, QuantParams(qk_bits=8, qk_format="int_e4m3"))
