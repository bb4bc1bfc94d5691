"""GPU parity of the MXFP4 Q/K format (SAGE_QK_MXFP4) against the oracle.

The FP4 microscaling of the SageAttention3 abstract, read as OCP MXFP4 (E2M1
codes, one E8M0 scale per 32 channels of a token) for the QK^T product; P~
and V stay FP8 as in the default path.  Bars as in test_gpu_parity.py: codes
(packed nibbles) and scale bytes bit-exact, Q/K means bit-exact, bias within
the split-bf16 bound, outputs within 2e-3 max|V| plus half an output ulp of the
oracle's emulation, and accuracy against exact attention at least the
emulation's (cos >= 0.999 and rel-L1 <= 0.02 where the emulation meets them).
"""
import numpy as np
import pytest

import oracle
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, scaled, make_inputs
from gpu_harness import run_sage, bits, bias_tolerance_ok, check_output, log, unpermute_v

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_fp16_d64": ("tiny", {}),
    "tiny_causal": ("tiny", {"causal": True}),
    "llm_prefill_ragged": ("llm_prefill", dict(B=1, H=2, N=1000)),
    "image_dit": ("image_dit", dict(B=1, H=2, N=777)),
    "target_small": ("target", dict(H=2, N=640)),
    "target_causal_small": ("target_causal", dict(H=2, N=700)),
    "d128_fp16": ("target", dict(dtype="fp16", H=2, N=513)),
    "d64_bf16": ("tiny", dict(dtype="bf16", N=300, H=3)),
    "batch2": ("llm_prefill", dict(B=2, H=3, N=260)),
    "n1": ("tiny", dict(N=1)),
    "long_tail": ("long_context", dict(H=2, N=1100)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_mxfp4_parity(case):
    name, kw = CASES[case]
    w = scaled(WORKLOADS[name], **kw)
    q, k, v = make_inputs(w)
    log(f"mxfp4 case {case}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    gpu = run_sage(q, k, v, w.dtype, w.causal, qk_format="mxfp4")
    p = QuantParams(qk_format="mxfp4")
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    for n in ("q_codes", "k_codes", "q_scale", "k_scale"):
        np.testing.assert_array_equal(gpu[n], qk[n], err_msg=n)
    for n in ("q_mean", "k_mean"):
        np.testing.assert_array_equal(bits(gpu[n]), bits(qk[n]), err_msg=n)
    np.testing.assert_array_equal(unpermute_v(gpu["v_codes"]), vq["v_codes"], err_msg="v codes")
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
