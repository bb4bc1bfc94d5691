"""GPU parity of INT4-range codes held in float formats: E4M3 bytes
(SAGE_QK_INT_E4M3) and packed FP6 E2M3 (SAGE_QK_INT_E2M3).

Every integer in [-7, 7] is exact in E4M3 and in E2M3, so the FP8 and FP6
matrix cores form the same integer S = q^ . k^ (fp32 partial sums of
integers below 2^24 are exact) as the INT8 matrix cores do for the int8-held
codes.  The bars: codes bit-exact against the oracle's bytes, scales and
means bit-exact, and the output bit-identical to the int8-held INT4-range
path on the same inputs (which test_gpu_parity.py holds to the oracle's
emulation); the emulation bar is checked here too.
"""
import numpy as np
import pytest

import oracle
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, scaled, make_inputs
from oracle.fp6 import e2m3_decode, unpack_slots
from gpu_harness import run_sage, bits, check_output, log, unpermute_v

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_fp16_d64": ("tiny", {}, "thread"),
    "tiny_causal_warp": ("tiny", {"causal": True}, "warp"),
    "image_dit_ragged": ("image_dit", dict(B=1, H=2, N=777), "thread"),
    "image_dit_block": ("image_dit", dict(B=1, H=2, N=600), "block"),
    "long_causal_tail": ("long_context_int4", dict(H=2, N=1100), "thread"),
    "target_fp16": ("target", dict(dtype="fp16", H=2, N=513), "thread"),
    "d64_bf16_batch2": ("tiny", dict(dtype="bf16", B=2, N=300, H=3), "warp"),
    "n1": ("tiny", dict(N=1), "thread"),
}


def _decode(codes, fmt):
    c = np.ascontiguousarray(codes).view(np.uint8)
    return oracle.e4m3_decode(c) if fmt == "int_e4m3" else e2m3_decode(unpack_slots(c))


@pytest.mark.parametrize("fmt", ["int_e4m3", "int_e2m3"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_int4_held_parity(case, fmt):
    name, kw, gran = CASES[case]
    w = scaled(WORKLOADS[name], **kw)
    q, k, v = make_inputs(w)
    log(f"int4 {fmt} case {case}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal} gran={gran}")
    gpu = run_sage(q, k, v, w.dtype, w.causal, qk_bits=4, gran=gran, qk_format=fmt)
    ref = run_sage(q, k, v, w.dtype, w.causal, qk_bits=4, gran=gran, qk_format="int")
    p = QuantParams(qk_bits=4, gran=gran, qk_format=fmt)
    qk, vq = oracle.quant_qk(q, k, p), oracle.quant_v(v, p)
    for n in ("q_codes", "k_codes"):
        np.testing.assert_array_equal(gpu[n].view(np.uint8), qk[n], err_msg=n)
    for n in ("q_scale", "k_scale", "q_mean", "k_mean"):
        np.testing.assert_array_equal(bits(gpu[n]), bits(qk[n]), err_msg=n)
    np.testing.assert_array_equal(unpermute_v(gpu["v_codes"]), vq["v_codes"], err_msg="v codes")
    # the same numbers as the int8-held codes, and the same output bits
    np.testing.assert_array_equal(_decode(gpu["k_codes"], fmt), ref["k_codes"].astype(np.float64))
    np.testing.assert_array_equal(np.asarray(gpu["out"]), np.asarray(ref["out"]), err_msg="output differs from the int8-held path")
    emul = oracle.emulate_attention(qk, vq, w.causal)
    nbad, maxerr, tol = check_output(gpu["out"], emul, v, w.dtype)
    log(f"  bit-identical to the int8-held path; vs emulation max err {maxerr:.3e} (tol {tol:.3e})")
    assert nbad == 0, f"{nbad} outputs beyond tolerance (max err {maxerr}, 2e-3 max|V| = {tol})"
