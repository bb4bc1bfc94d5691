"""Pins of the MXFP4 codec and quantiser (oracle/fp4.py) and of the emulation's
MXFP4 score path.

E2M1 and E8M0 follow the OCP microscaling format definition (1 sign, 2
exponent bits with bias 1, 1 mantissa bit; scale byte e = 2^(e - 127)); the
block exponent rule (smallest s with 6 * 2^s >= amax) is a reading
of the SageAttention3 abstract's FP4 microscaling, stated in oracle/fp4.py.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.fp4 as f4
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled

# code -> value, written out from the format definition
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_decode_table():
    got = f4.e2m1_decode(np.arange(16))
    assert np.array_equal(got, E2M1_TABLE)
    assert np.array_equal(np.signbit(got), [c >= 8 for c in range(16)])


# Hand-worked roundings: nearest magnitude, a tie to the code with mantissa
# bit 0, saturation at 6, sign kept.
LANDMARKS = [(0.0, 0), (0.2499999, 0), (0.25, 0), (0.2500001, 1), (0.5, 1), (0.7499999, 1), (0.75, 2),
             (1.25, 2), (1.2500001, 3), (1.75, 4), (2.4999998, 4), (2.5, 4), (2.5000002, 5), (3.5, 6), (4.9999995, 6),
             (5.0, 6), (5.0000005, 7), (6.0, 7), (7.0, 7), (1e30, 7), (-0.0, 8), (-1e-8, 8), (-0.75, 10), (-5.0, 14),
             (-5.5, 15), (-100.0, 15)]


@pytest.mark.parametrize("x,code", LANDMARKS)
def test_encode_landmarks(x, code):
    assert int(f4.e2m1_encode(np.float32(x))) == code


def _brute_encode(x: float) -> int:
    """Nearest of the 8 magnitudes by exhaustive search, ties to the even code, saturating."""
    a = min(abs(x), 6.0)
    best = min(range(8), key=lambda c: (abs(E2M1_TABLE[c] - a), c % 2))
    return best | (8 if math.copysign(1.0, x) < 0 else 0)


def test_encode_matches_brute_force():
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.uniform(-8, 8, 4000), rng.standard_normal(2000) * 0.3,
                         np.arange(-7, 7.01, 0.125)]).astype(np.float32)
    got = f4.e2m1_encode(xs)
    want = np.array([_brute_encode(float(x)) for x in xs])
    assert np.array_equal(got, want)


def test_round_trip_of_every_code():
    vals = f4.e2m1_decode(np.arange(16)).astype(np.float32)
    assert np.array_equal(f4.e2m1_encode(vals), np.arange(16))


EXPONENTS = [(6.0, 0), (6.0000005, 1), (4.0, 0), (3.0, -1), (3.0000002, 0), (1.0, -2), (1.5, -2), (0.75, -3),
             (12.0, 1), (0.0, -127), (1e-45, -127), (2.0 ** -120, -122), (3.0e38, 126)]


@pytest.mark.parametrize("amax,s", EXPONENTS)
def test_block_exponent_examples(amax, s):
    assert int(f4.block_exponent(np.float32(amax))) == s


def test_block_exponent_is_the_smallest_cover():
    rng = np.random.default_rng(4)
    a = np.exp(rng.uniform(-40, 40, 20000)).astype(np.float32)
    s = f4.block_exponent(a)
    a64 = a.astype(np.float64)
    assert np.all(6.0 * np.exp2(s.astype(np.float64)) >= a64)
    assert np.all(6.0 * np.exp2(s.astype(np.float64) - 1) < a64)


def _rows(n=40, d=128, seed=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, 1, n, d)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (1, 1, n, 1)))
    x[0, 0, 3, :32] = 0.0                          # an all-zero block
    x[0, 0, 4, 40] = 37.0                          # an outlier
    return x


def test_mx_quantiser_invariants():
    x = _rows()
    valid = np.arange(40) < 37                     # three padded rows
    codes, scale = f4.mx_quantize_rows(x, valid)
    assert codes.shape == (1, 1, 40, 128) and scale.shape == (1, 1, 40, 4)
    assert not codes[..., 37:, :].any() and not scale[..., 37:, :].any()
    dec = f4.mx_decode_rows(codes, scale)
    blocks = x[..., :37, :].reshape(1, 1, 37, 4, 32).astype(np.float64)
    s = scale[..., :37, :].astype(np.float64) - 127
    amax = np.abs(blocks).max(axis=-1)
    nz = amax > 0
    # no element saturates, and the block maximum lands on 3, 4 or 6 (times 2^s)
    assert np.all(amax[nz] <= 6 * np.exp2(s[nz]))
    top = np.abs(dec[..., :37, :].reshape(1, 1, 37, 4, 32)).max(axis=-1)
    assert np.all(top[nz] >= 3 * np.exp2(s[nz]))
    # each element is within half a local gap of its value (largest gap 2, at 4..6)
    err = np.abs(dec[..., :37, :].reshape(1, 1, 37, 4, 32) - blocks)
    assert np.all(err <= 1.0 * np.exp2(s)[..., None] + 1e-30)
    assert scale[0, 0, 3, 0] == 0 and not codes[0, 0, 3, :32].any()   # zero block: scale 2^-127, zero codes


def test_pack_nibbles_order():
    c = np.arange(16, dtype=np.uint8)
    p = f4.pack_nibbles(c)
    assert list(p) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(f4.unpack_nibbles(p), c)


FP4_SLIPS = {
    "exponent rounded down (OCP shared-exponent rule)": ("s = np.where(m <= (1 << 22), e - 2, e - 1)", "s = e - 2"),
    "ties away from zero": ("(d_hi == d_lo) & (hi % 2 == 0)", "(d_hi == d_lo)"),
    "sign dropped": ("np.where(np.signbit(x32), code | np.uint8(0x8), code)", "np.where(np.signbit(x32), code, code)"),
    "subnormal code skipped": ("_MAG = np.array([0.0, 0.5, 1.0,", "_MAG = np.array([0.0, 1.0, 1.0,"),
}


@pytest.mark.parametrize("name", sorted(FP4_SLIPS))
def test_planted_fp4_slips_are_caught(name, monkeypatch):
    import inspect
    import textwrap
    old, new = FP4_SLIPS[name]
    mod_src = textwrap.dedent(inspect.getsource(f4))
    assert mod_src.count(old) == 1, f"mutation anchor for {name!r} not found once"
    ns = {}
    exec(compile(mod_src.replace(old, new), "<planted>", "exec"), ns)
    for fn in ("e2m1_encode", "block_exponent", "mx_quantize_rows"):
        monkeypatch.setattr(f4, fn, ns[fn])
    caught = False
    for test in (test_encode_matches_brute_force, test_block_exponent_is_the_smallest_cover, test_mx_quantiser_invariants):
        try:
            with np.errstate(all="ignore"):
                test()
        except (AssertionError, IndexError, ValueError):
            caught = True
    for x, code in LANDMARKS:
        try:
            if int(f4.e2m1_encode(np.float32(x))) != code:
                caught = True
        except (IndexError, ValueError):
            caught = True
    assert caught, f"planted slip {name!r} went unnoticed"


@pytest.mark.parametrize("causal", [False, True])
def test_mxfp4_score_path_equals_plain_softmax(causal):
    """With 16-bit P~V (no FP8 anywhere) the tiled emulation on MXFP4 codes must
    equal the plain softmax of s = (Q^ K^T + dS) sm_scale, with Q^ and K^ the
    decoded MXFP4 rows and dS the smoothing bias, up to the 16-bit rounding of
    the weights: |O - O_plain| <= u max|V| (u = 2^-11 for fp16)."""
    w = scaled(WORKLOADS["tiny"], N=300)            # fp16, d = 64, ragged
    q, k, v = make_inputs(w)
    p = QuantParams(qk_format="mxfp4", pv="fp16")
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    em = oracle.emulate_attention(qk, vq, causal)
    N, scale = w.N, 1 / math.sqrt(w.d)
    for h in range(w.H):
        qd, kd = qk["q_values"][0, h, :N], qk["k_values"][0, h, :N]
        bias = np.repeat(qk["bias"][0, h].astype(np.float64), 128, axis=0)[:N, :N]
        s = (qd @ kd.T + bias) * scale
        if causal:
            s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
        pmat = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (pmat / pmat.sum(axis=1, keepdims=True)) @ v[0, h].astype(np.float64)
        assert np.abs(em[0, h] - ref).max() <= 2.0 ** -11 * np.abs(v).max() * (1 + 1e-3) + 1e-6
