"""Pins of the E2M3 codec and the slot packing (oracle/fp6.py), and of the
E2M3-held INT4-range format of the oracle's quantiser.

E2M3 (1 sign, 2 exponent bits with bias 1, 3 mantissa bits) follows the OCP
microscaling FP6 definition; the slot packing is the FP6 operand layout of the
gfx950 64-deep matrix product (value i of a lane's 32 at bits 6 i .. 6 i + 5,
lane halves pairing channel for channel), stated in oracle/fp6.py.
"""
import inspect
import textwrap

import numpy as np
import pytest

import oracle
import oracle.fp6 as f6
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled

# magnitudes of codes 0..31 written out: subnormals m/8, then 1..1.875, 2..3.75, 4..7.5
MAGS = [i / 8 for i in range(8)] + [1 + i / 8 for i in range(8)] + [2 + i / 4 for i in range(8)] + \
       [4 + i / 2 for i in range(8)]
# E2M3 codes of the integers 0..7, worked by hand: 1 = 1.0 x 2^0 -> 0 01 000 = 8; 3 = 1.5 x 2^1 -> 0 10 100 = 20;
# 5 = 1.25 x 2^2 -> 0 11 010 = 26; 7 = 1.75 x 2^2 -> 0 11 110 = 30
INT_CODES = [0, 8, 16, 20, 24, 26, 28, 30]


def test_decode_table():
    got = f6.e2m3_decode(np.arange(64))
    assert np.array_equal(got[:32], MAGS)
    assert np.array_equal(got[32:], -np.array(MAGS))


def test_integer_codes():
    ints = np.arange(-7, 8).astype(np.float32)
    want = np.array([INT_CODES[abs(int(i))] | (0x20 if i < 0 else 0) for i in ints], np.uint8)
    np.testing.assert_array_equal(f6.e2m3_encode(ints), want)
    np.testing.assert_array_equal(f6.e2m3_decode(want), ints)


def test_encode_matches_brute_force_and_round_trips():
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.uniform(-9, 9, 3000), np.arange(-8, 8.01, 1 / 16)]).astype(np.float32)
    table = np.array(MAGS)
    for x, c in zip(xs, f6.e2m3_encode(xs)):
        a = min(abs(float(x)), 7.5)
        best = min(range(32), key=lambda k: (abs(table[k] - a), k % 2))
        assert c == (best | (0x20 if np.signbit(x) else 0)), x
    np.testing.assert_array_equal(f6.e2m3_encode(f6.e2m3_decode(np.arange(64)).astype(np.float32)),
                                  np.where(np.arange(64) == 32, 32, np.arange(64)))


def test_slot_packing_hand_examples():
    """One code at a time in a d = 64 row: where its six bits land, worked by hand."""
    cases = {   # channel: (row byte, value at that byte[, next byte, value])
        0: [(0, 0x3F)],                      # slot (0,0) value 0: bits 0..5
        1: [(0, 0xC0), (1, 0x0F)],           # slot (0,0) value 1: bits 6..11
        16: [(16, 0x3F)],                    # slot (0,1) value 0 at byte 16 (4 j + h = 1)
        32: [(12, 0x3F)],                    # slot (0,0) value 16: bits 96..101, slot byte 12
        40: [(34, 0x3F)],                    # slot (0,0) value 24: bits 144..149, slot byte 18 -> 16 * 2 + 2
        48: [(28, 0x3F)],                    # slot (0,1) value 16: slot byte 12 -> 16 * 1 + 12
        63: [(55, 0xFC)],                    # slot (0,1) value 31: bits 186..191, slot byte 23 -> 16 * 3 + 7
    }
    for ch, where in cases.items():
        codes = np.zeros(64, np.uint8)
        codes[ch] = 0x3F
        row = f6.pack_slots(codes)
        want = np.zeros(64, np.uint8)
        for (byte, val) in where:
            want[byte] = val
        np.testing.assert_array_equal(row, want, err_msg=f"channel {ch}")


def test_pack_round_trip_and_padding():
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 64, (3, 5, 128)).astype(np.uint8)
    packed = f6.pack_slots(codes)
    np.testing.assert_array_equal(f6.unpack_slots(packed), codes)
    for j in range(2):
        for h in range(2):
            pad = 16 * (4 * j + 2 + h) + 8
            assert not packed[..., pad:pad + 8].any()


@pytest.mark.parametrize("gran", ["thread", "warp", "block"])
def test_int_e2m3_holds_the_int4_codes(gran):
    w = scaled(WORKLOADS["image_dit"], B=1, H=2, N=300)
    q, k, v = make_inputs(w)
    pi = QuantParams(qk_bits=4, gran=gran)
    pe = QuantParams(qk_bits=4, gran=gran, qk_format="int_e2m3")
    a, b = oracle.quant_qk(q, k, pi), oracle.quant_qk(q, k, pe)
    for n in ("q_codes", "k_codes"):
        np.testing.assert_array_equal(f6.e2m3_decode(f6.unpack_slots(b[n])), a[n].astype(np.float64), err_msg=n)
    for n in ("q_scale", "k_scale", "q_mean", "k_mean", "bias"):
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
    vq = oracle.quant_v(v, pi)
    for causal in (False, True):
        np.testing.assert_array_equal(oracle.emulate_attention(a, vq, causal), oracle.emulate_attention(b, vq, causal))


SLIPS = {
    "exponent bias 0": ("np.exp2(e.astype(np.float64) - 1.0)", "np.exp2(e.astype(np.float64))"),
    "halves swapped": ("64 * j + 16 * h + i if i < 16", "64 * j + 16 * (1 - h) + i if i < 16"),
    "bits big-endian": ("packed[..., bit // 8] |= (((vals[..., i] >> np.uint64(b))",
                        "packed[..., 23 - bit // 8] |= (((vals[..., i] >> np.uint64(b))"),
}


@pytest.mark.parametrize("name", sorted(SLIPS))
def test_planted_slips_are_caught(name, monkeypatch):
    old, new = SLIPS[name]
    src = textwrap.dedent(inspect.getsource(f6))
    assert src.count(old) == 1, name
    ns = {}
    exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
    for fn in ("e2m3_decode", "e2m3_encode", "slot_channels", "pack_slots", "unpack_slots"):
        monkeypatch.setattr(f6, fn, ns[fn])
    monkeypatch.setattr(f6, "_MAG", ns["_MAG"])
    caught = False
    for test in (test_decode_table, test_integer_codes, test_slot_packing_hand_examples):
        try:
            test()
        except AssertionError:
            caught = True
    assert caught, f"planted slip {name!r} went unnoticed"
