"""GPU parity of the 16-bit P~V mode (SAGE_PV_F16) against the oracle.

The first SageAttention's setting, which the SageAttention2 abstract builds
on: the same Q, K quantisation and online softmax as the FP8 path, P~ rounded
to the input's 16-bit type and V used as given on the bf16/fp16 matrix cores.
Bars (as in test_gpu_parity.py): Q, K codes, scales and means bit-exact; the
V buffer bit-equal to the input (in the documented key order), scale 1, mean
0; bias within the split-bf16 bound; outputs within 2e-3 max|V| plus half an
output ulp of the oracle's emulation of this mode; against exact attention at
least as accurate as the emulation (cos >= 0.999, rel-L1 <= 0.02 where it
meets them).
"""
import numpy as np
import pytest

import oracle
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, scaled, make_inputs
from gpu_harness import (run_sage, bits, bias_tolerance_ok, check_output, log, unpermute_v16, half_bits)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_fp16_d64": ("tiny", {}),
    "tiny_causal": ("tiny", {"causal": True}),
    "llm_prefill_ragged": ("llm_prefill", dict(B=1, H=2, N=1000)),
    "image_dit_int4": ("image_dit", dict(B=1, H=2, N=777)),
    "target_small": ("target", dict(H=2, N=640)),
    "target_causal_small": ("target_causal", dict(H=2, N=700)),
    "d128_fp16": ("target", dict(dtype="fp16", H=2, N=513)),
    "d64_bf16": ("tiny", dict(dtype="bf16", N=300, H=3)),
    "batch2": ("llm_prefill", dict(B=2, H=3, N=260)),
    "n1": ("tiny", dict(N=1)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_pv16_parity(case):
    name, kw = CASES[case]
    w = scaled(WORKLOADS[name], **kw)
    q, k, v = make_inputs(w)
    log(f"pv16 case {case}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal} bits={w.qk_bits}")
    gpu = run_sage(q, k, v, w.dtype, w.causal, w.qk_bits, w.gran, pv="f16")
    p = QuantParams(qk_bits=w.qk_bits, gran=w.gran, pv=w.dtype)
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    for n in ("q_codes", "k_codes"):
        np.testing.assert_array_equal(gpu[n], qk[n], err_msg=n)
    for n in ("q_scale", "k_scale", "q_mean", "k_mean"):
        np.testing.assert_array_equal(bits(gpu[n]), bits(qk[n]), err_msg=n)
    np.testing.assert_array_equal(unpermute_v16(gpu["v_codes"]), half_bits(vq["v_values"], w.dtype), err_msg="V")
    assert (gpu["v_scale"] == 1).all() and not gpu["v_mean"].any()
    ok, worst = bias_tolerance_ok(gpu["bias"], qk["bias"], qk["q_mean"], qk["k_smoothed"])
    assert ok, f"bias error {worst} of the bound"
    emul = oracle.emulate_attention(qk, vq, w.causal)
    nbad, maxerr, tol = check_output(gpu["out"], emul, v, w.dtype)
    assert nbad == 0, f"{nbad} outputs beyond tolerance (max err {maxerr}, 2e-3 max|V| = {tol})"
    ex = oracle.exact_attention(q, k, v, w.causal)
    m_gpu, m_em = oracle.compare(ex, gpu["out"]), oracle.compare(ex, emul)
    log(f"  vs emulation max err {maxerr:.3e} (tol {tol:.3e}); vs exact gpu {m_gpu} emul {m_em}")
    assert m_gpu["cos"] >= min(0.999, m_em["cos"] - 2e-4)
    assert m_gpu["rel_l1"] <= max(0.02, m_em["rel_l1"] + 0.003)


def test_pv16_more_accurate_than_fp8_pv():
    """The ablation the pages draw between SageAttention and SageAttention2:
    with the same QK quantisation the 16-bit P~V is closer to exact attention
    than the FP8 one, on both the GPU and the emulation."""
    w = scaled(WORKLOADS["target"], H=2, N=1024)
    q, k, v = make_inputs(w)
    ex = oracle.exact_attention(q, k, v, w.causal)
    res = {}
    for pv in ("fp8", "f16"):
        gpu = run_sage(q, k, v, w.dtype, w.causal, w.qk_bits, w.gran, pv=pv, download=())
        res[pv] = oracle.compare(ex, gpu["out"])
    log(f"  vs exact: fp8 P~V {res['fp8']}; 16-bit P~V {res['f16']}")
    assert res["f16"]["rel_l1"] < res["fp8"]["rel_l1"]
    assert res["f16"]["cos"] > res["fp8"]["cos"]
