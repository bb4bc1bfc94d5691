"""Pins of the attention backward oracle (oracle/backward.py).

Exact float64 gradients: central finite differences of the exact forward
(the definition of the derivative), and the invariants of softmax attention
(shifting every key together moves nothing, so the key gradients sum to zero;
rows of P sum to one, so the value gradients sum to the summed dO; identical
value rows make O independent of Q and K).

The 8-bit emulation: with every quantiser off (and the exact O in D) it must
equal the exact gradients up to fp32 rounding; each quantiser alone stays
within its E4M3 rounding window; the power-of-two group exponent is checked
against hand-worked values and its definition; planted slips are caught.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import backward as ob
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled

U8 = 2.0 ** -4     # E4M3 unit roundoff


def _loss(q, k, v, do, causal):
    return float((oracle.exact_attention(q, k, v, causal) * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_exact_gradients_match_finite_differences(causal):
    rng = np.random.default_rng(21)
    q, k, v, do = (rng.standard_normal((1, 1, 6, 3)) for _ in range(4))
    dq, dk, dv = ob.exact_attention_grad(q, k, v, do, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            up = _loss(q, k, v, do, causal)
            x[idx] = old - h
            dn = _loss(q, k, v, do, causal)
            x[idx] = old
            assert abs((up - dn) / (2 * h) - g[idx]) <= 1e-7 * (1 + abs(g[idx]))


def test_exact_gradients_brute_force_tiny():
    # N = 2, d = 1, non-causal, written out: z = c q k, p = softmax(z) per row.
    q, k, v, do = (np.array([[[[a], [b]]]], np.float64) for a, b in ((0.3, -1.2), (0.8, 0.1), (2.0, -1.0),
                                                                       (0.5, 1.5)))
    c = 1.0
    dq, dk, dv = ob.exact_attention_grad(q, k, v, do, False, sm_scale=c)
    for i in range(2):
        z = [c * q[0, 0, i, 0] * k[0, 0, j, 0] for j in range(2)]
        e = [math.exp(t) for t in z]
        p = [t / sum(e) for t in e]
        o = sum(p[j] * v[0, 0, j, 0] for j in range(2))
        dpij = [do[0, 0, i, 0] * v[0, 0, j, 0] for j in range(2)]
        D = do[0, 0, i, 0] * o
        ds = [p[j] * (dpij[j] - D) for j in range(2)]
        assert abs(dq[0, 0, i, 0] - c * sum(ds[j] * k[0, 0, j, 0] for j in range(2))) <= 1e-14
    # dV_j = sum_i P_ij dO_i
    P = np.exp(c * q[0, 0] @ k[0, 0].T)
    P /= P.sum(axis=1, keepdims=True)
    assert np.abs(dv[0, 0] - P.T @ do[0, 0]).max() <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_exact_gradient_invariants(causal):
    rng = np.random.default_rng(22)
    q, k, v, do = (rng.standard_normal((1, 2, 30, 8)) for _ in range(4))
    dq, dk, dv = ob.exact_attention_grad(q, k, v, do, causal)
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12                       # key shift invariance
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() <= 1e-12      # rows of P sum to 1
    vc = np.repeat(v[:, :, :1], 30, axis=2)                           # O = v_0 for every row
    dq0, dk0, _ = ob.exact_attention_grad(q, k, vc, do, causal)
    assert np.abs(dq0).max() <= 1e-12 and np.abs(dk0).max() <= 1e-12


def test_e8m0_exponent_examples_and_definition():
    cases = {448.0: 0, 449.0: 1, 224.0: -1, 224.5: 0, 1.0: -8, 1.75: -8, 1.7500001: -7, 0.0: -127, 3e-39: -127}
    for amax, e in cases.items():
        assert int(ob.e8m0_exponent(np.float32(amax))) == e, amax
    rng = np.random.default_rng(23)
    xs = np.exp(rng.uniform(-60, 60, 20000)).astype(np.float32)
    es = ob.e8m0_exponent(xs)
    # smallest e with 448 2^e >= amax, by the definition
    assert np.all(448.0 * np.exp2(es.astype(np.float64)) >= xs)
    assert np.all(448.0 * np.exp2(es.astype(np.float64) - 1) < xs)


def test_mx8_groups_follow_the_axis():
    x = np.zeros((64, 128), np.float32)
    x[5, 7] = 300.0          # a large entry: its group gets the scale 2^0
    x[5, 70] = 0.0009        # same row, other 64-column group
    x[40, 7] = 0.0009        # same column, other row
    # at scale 2^0 the smallest E4M3 step is 2^-9, and 0.0009 < 2^-10 rounds to 0
    vals_r, e_r = ob.mx8_values(x, axis=1)      # groups of 64 columns per row
    assert e_r.shape == (64, 2) and e_r[5, 0] == 0 and e_r[40, 0] == ob.e8m0_exponent(np.float32(0.0009))
    assert abs(vals_r[40, 7] - 0.0009) <= U8 * 0.0009 and abs(vals_r[5, 70] - 0.0009) <= U8 * 0.0009
    vals_c, e_c = ob.mx8_values(x, axis=0)      # groups of 64 rows per column
    assert e_c.shape == (128, 1) and e_c[7, 0] == 0
    assert vals_c[40, 7] == 0.0 and vals_c[5, 7] == 288.0   # 300 -> nearest E4M3 (spacing 32 in [256, 448])
    assert abs(vals_c[5, 70] - 0.0009) <= U8 * 0.0009


def _setup(name, N, causal, seed=31, quantized=True):
    w = scaled(WORKLOADS[name], B=1, H=2, N=N)
    q, k, v = make_inputs(w)
    do = np.random.default_rng(seed).standard_normal(q.shape).astype(np.float32)
    return w, q, k, v, do


def _identity_error(name="image_dit", N=300, causal=False, block=None):
    w, q, k, v, do = _setup(name, N, causal)
    o_id, lse, qk, vq = ob.forward_with_lse(q, k, v, causal, w.dtype, quantized=False)
    o_ex = oracle.exact_attention(q, k, v, causal)
    ctx = ob.prepare(q, k, v, do, o_ex, lse, qk, causal, codecs=())
    em = ob.emulate_backward(ctx)
    ex = ob.exact_attention_grad(q, k, v, do, causal)
    return [float(np.abs(g - e).max() / np.abs(e).max()) for g, e in zip(em, ex)]


@pytest.mark.parametrize("name,N,causal", [("image_dit", 300, False), ("llm_prefill", 260, True),
                                           ("target", 200, False), ("tiny", 130, True)])
def test_backward_without_quantisation_is_exact(name, N, causal):
    errs = _identity_error(name, N, causal)
    assert max(errs) <= 2e-5, errs


def _codec_error(codecs, causal, name="image_dit", N=300):
    """Each gradient's |emulated - exact-path| against an elementwise bound of
    the one quantiser switched on (E4M3 rounding of its operand)."""
    w, q, k, v, do = _setup(name, N, causal)
    o_id, lse, qk, vq = ob.forward_with_lse(q, k, v, causal, w.dtype, quantized=False)
    o_ex = oracle.exact_attention(q, k, v, causal)
    base = ob.prepare(q, k, v, do, o_ex, lse, qk, causal, codecs=())
    ref = ob.emulate_backward(base)
    ctx = ob.prepare(q, k, v, do, o_ex, lse, qk, causal, codecs=codecs)
    return ref, ob.emulate_backward(ctx), base


@pytest.mark.parametrize("causal", [False, True])
def test_p_codec_window(causal):
    """P to E4M3 (scale 1/P_r) moves only dV: each weight by at most u P + 2^-10 / P_r."""
    ref, em, base = _codec_error({"p"}, causal)
    assert np.array_equal(ref[0], em[0]) and np.array_equal(ref[1], em[1])
    N = base["N"]
    err = np.abs(em[2] - ref[2])
    P_sum = np.zeros_like(err)
    for b in range(1):
        for h in range(2):
            for kb in range(base["n_pad"] // 128):
                cols = kb * 128 + np.arange(128)
                for q0 in range(0, base["n_pad"], 128):
                    rows = q0 + np.arange(128)
                    P, _ = ob._tile(base, b, h, rows, cols)
                    bound = (U8 * P.astype(np.float64) + (P > 0) * 2.0 ** -10 / base["p_range"]).T @ np.abs(
                        base["do"][b, h, rows])
                    sel = cols < N
                    P_sum[b, h, cols[sel]] += bound[sel]
    assert np.all(err <= P_sum * (1 + 1e-6) + 1e-12)
    assert err.max() >= U8 / 64 * np.abs(ref[2]).max()       # the weights really were rounded


def _ds_bounds(base):
    """Elementwise bounds on the dQ and dK errors of the dS quantiser alone:
    an element of a group with exponent e moves by at most max(u |dS|,
    2^-10 2^e); dQ groups run along the keys of a query row, dK groups along
    the queries of a key (64 each, aligned)."""
    n_pad, N, c = base["n_pad"], base["N"], base["c"]
    bq = np.zeros((1, 2, n_pad, base["d"]))
    bk = np.zeros_like(bq)
    for h in range(2):
        for qb in range(n_pad // 128):
            rows = qb * 128 + np.arange(128)
            for kb in range(n_pad // 128):
                cols = kb * 128 + np.arange(128)
                _, dS = ob._tile(base, 0, h, rows, cols)
                a = np.abs(dS.astype(np.float64))
                e_row = ob.e8m0_exponent(np.abs(dS).reshape(128, 2, 64).max(axis=2))       # [query, key group]
                e_col = ob.e8m0_exponent(np.abs(dS).reshape(2, 64, 128).max(axis=1))       # [query group, key]
                b_q = np.maximum(U8 * a, 2.0 ** -10 * np.exp2(np.repeat(e_row, 64, axis=1).astype(np.float64)))
                b_k = np.maximum(U8 * a, 2.0 ** -10 * np.exp2(np.repeat(e_col, 64, axis=0).astype(np.float64)))
                b_q[a == 0] = 0
                b_k[a == 0] = 0
                bq[0, h, rows] += c * b_q @ np.abs(base["k"][0, h, cols])
                bk[0, h, cols] += c * b_k.T @ np.abs(base["q"][0, h, rows])
    return bq[:, :, :N], bk[:, :, :N]


@pytest.mark.parametrize("causal", [False, True])
def test_ds_codec_window(causal):
    """dS to E4M3 with power-of-two group scales (the dQ groups along keys, the
    dK groups along queries) moves only dQ and dK, each element within its
    propagated rounding bound, and by enough to show the rounding happened."""
    ref, em, base = _codec_error({"ds"}, causal)
    assert np.array_equal(ref[2], em[2])
    bq, bk = _ds_bounds(base)
    for g_ref, g_em, bound in ((ref[0], em[0], bq), (ref[1], em[1], bk)):
        err = np.abs(g_em - g_ref)
        assert np.all(err <= bound * (1 + 1e-6) + 1e-12), float((err / (bound + 1e-30)).max())
        assert err.max() >= U8 / 64 * np.abs(g_ref).max()


def _axis_case_ok():
    """dq_block must group dS along keys (per query row), dkdv_block along
    queries (per key).  With K' = Q = I (d = 128), c = 1 and every other
    quantiser off, the blocks return the quantised dS itself (dQ) and its
    transpose (dK); a large entry flushes the small ones of its own group only."""
    import unittest.mock as um
    dS = np.zeros((128, 128), np.float32)
    dS[5, 7], dS[40, 7], dS[5, 70] = 300.0, 0.0009, 0.0009
    eye = np.eye(128)[None, None]
    ctx = dict(q=eye, k=eye, v=np.zeros_like(eye), do=np.zeros_like(eye), N=128, n_pad=128, d=128, causal=False,
               c=1.0, p_range=448.0, codecs=frozenset({"ds"}))
    fake = lambda c_, b, h, rows, cols: (np.zeros((128, 128), np.float32), dS)   # noqa: E731
    with um.patch.dict(ob.dq_block.__globals__, {"_tile": fake}), \
            um.patch.dict(ob.dkdv_block.__globals__, {"_tile": fake}):
        dq = ob.dq_block(ctx, 0, 0, 0)
        dk, _ = ob.dkdv_block(ctx, 0, 0, 0)
    row_ok = abs(dq[40, 7] - 0.0009) <= U8 * 0.0009 and abs(dq[5, 70] - 0.0009) <= U8 * 0.0009
    col_ok = dk[7, 40] == 0.0 and abs(dk[70, 5] - 0.0009) <= U8 * 0.0009
    return bool(row_ok and col_ok and dq[5, 7] == 288.0 and dk[7, 5] == 288.0)


def test_dq_and_dk_group_ds_along_their_reduction_axes():
    assert _axis_case_ok()


def test_quantised_backward_accuracy():
    """All five 8-bit products together stay near the exact gradients on the
    image-DiT recipe (V with channel means), as the forward does."""
    w, q, k, v, do = _setup("image_dit", 300, False)
    o, lse, qk, vq = ob.forward_with_lse(q, k, v, False, w.dtype, QuantParams(qk_bits=8))
    em = ob.emulate_backward(ob.prepare(q, k, v, do, o, lse, qk, False))
    ex = ob.exact_attention_grad(q, k, v, do, False)
    for g, e in zip(em, ex):
        m = oracle.compare(e, g)
        assert m["cos"] >= 0.998 and m["rel_l1"] <= 0.06, m


def test_forward_lse_normalises_p():
    """2^(s - L) over a row's keys sums to one (L from the forward's m and l)."""
    w, q, k, v, do = _setup("llm_prefill", 300, True)
    o, lse, qk, vq = ob.forward_with_lse(q, k, v, True, w.dtype, quantized=False)
    ctx = ob.prepare(q, k, v, do, o, lse, qk, True, codecs=())
    for qb in range(3):
        rows = qb * 128 + np.arange(128)
        tot = sum(ob._tile(ctx, 0, 0, rows, kb * 128 + np.arange(128))[0].astype(np.float64).sum(axis=1)
                  for kb in range(3))
        valid = rows < 300
        assert np.abs(tot[valid] - 1).max() <= 1e-5


# Plausible slips planted into copies of the backward blocks (source
# substitution); the identity-codec check against the exact gradients, or a
# window, must catch each.
SLIPS = {
    "D dropped": ("dS = np.where(valid, P.astype(np.float64) * t.astype(np.float64), 0.0)",
                  "dS = np.where(valid, P.astype(np.float64) * dP.astype(np.float64), 0.0)"),
    "P against the row max, not L": ("np.exp2(s.astype(np.float64) - L[:, None])",
                                     "np.exp2(s.astype(np.float64) - s.max(axis=1, keepdims=True))"),
    "causal mask off by one": ("valid &= cols[None, :] <= rows[:, None]", "valid &= cols[None, :] < rows[:, None]"),
    "dK without the softmax scale": ("return ctx[\"c\"] * dk * qs[None, :], dv * dos[None, :]",
                                     "return dk * qs[None, :], dv * dos[None, :]"),
    "dS not transposed for dK": ("dk += w.T @ qv", "dk += w @ qv"),
    "dV from dS": ("dv += pw.T @ dov", "dv += dS.astype(np.float64).T @ dov"),
    "dQ groups along queries": ("w = mx8_values(dS, axis=1)[0] if", "w = mx8_values(dS, axis=0)[0] if"),
}


@pytest.mark.parametrize("name", sorted(SLIPS))
def test_planted_backward_slips_are_caught(name, monkeypatch):
    import inspect
    import textwrap
    old, new = SLIPS[name]
    ns = dict(vars(ob))
    found = 0
    for fn in ("_tile", "dq_block", "dkdv_block"):
        src = textwrap.dedent(inspect.getsource(getattr(ob, fn)))
        if old in src:
            found += src.count(old)
            exec(compile(src.replace(old, new), "<planted>", "exec"), ns)
            monkeypatch.setattr(ob, fn, ns[fn])
    assert found == 1, f"mutation anchor for {name!r} found {found} times"
    for f in ("_tile", "dq_block", "dkdv_block"):      # the planted copies call each other through ns
        ns[f] = getattr(ob, f)
    with np.errstate(all="ignore"):
        caught = max(_identity_error("llm_prefill", 260, True)) > 1e-3 or \
            max(_identity_error("image_dit", 300, False)) > 1e-3
        if not caught:
            try:
                test_ds_codec_window(False)
                test_ds_codec_window(True)
            except AssertionError:
                caught = True
        caught = caught or not _axis_case_ok()
    assert caught, f"planted slip {name!r} went unnoticed"
