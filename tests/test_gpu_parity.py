"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (derived from the arithmetic of each step):
  * codes, scales and means: bit-exact against the oracle's fp32 emulation;
  * bias dS: |err| <= 2^-14 sum_c |mu_Q,c| |K'_jc| (bf16 hi/lo split products);
  * output: |O_gpu - O_emul| <= 2e-3 max|V| + half an fp16/bf16 ulp of O;
  * against exact fp64 attention: cos >= 0.999 and rel-L1 <= 0.02 where the
    emulation itself meets them; otherwise the GPU must be no worse than the
    emulation (plus a small margin).  FP8 P~ and FP8 V each cost about 0.025
    rel-L1 on zero-mean random V, so that bar is a property of the method.
"""
import numpy as np
import pytest

import oracle
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled
from gpu_harness import (run_sage, assert_quant_bit_exact, bias_tolerance_ok, check_output, log)

pytestmark = pytest.mark.gpu


def _check_case(w, gran=None, smooth=(True, True, True), p_range=448.0, v_range=448.0, layout="bhnd"):
    q, k, v = make_inputs(w)
    return _check_inputs(w, q, k, v, gran, smooth, p_range, v_range, layout)


def _check_inputs(w, q, k, v, gran=None, smooth=(True, True, True), p_range=448.0, v_range=448.0, layout="bhnd",
                  vs_exact=True):
    gran = gran or w.gran
    log(f"case {w.name} B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal} bits={w.qk_bits} "
        f"gran={gran} smooth={smooth} pr={p_range} vr={v_range} layout={layout}")
    gpu = run_sage(q, k, v, w.dtype, w.causal, w.qk_bits, gran, smooth, p_range, v_range, layout)
    p = QuantParams(qk_bits=w.qk_bits, gran=gran, smooth_q=smooth[0], smooth_k=smooth[1], smooth_v=smooth[2],
                    p_range=p_range, v_range=v_range)
    qk = oracle.quant_qk(q, k, p)
    vq = oracle.quant_v(v, p)
    assert_quant_bit_exact(gpu, qk, vq)
    ok, worst = bias_tolerance_ok(gpu["bias"], qk["bias"], qk["q_mean"], qk["k_smoothed"])
    assert ok, f"bias error {worst} of the bound scale"
    emul = oracle.emulate_attention(qk, vq, w.causal, p_range=p_range)
    nbad, maxerr, tol = check_output(gpu["out"], emul, v, w.dtype)
    assert nbad == 0, f"{nbad} outputs beyond tolerance (max err {maxerr}, 2e-3 max|V| = {tol})"
    if not vs_exact:
        return gpu
    ex = oracle.exact_attention(q, k, v, w.causal)
    m_gpu, m_em = oracle.compare(ex, gpu["out"]), oracle.compare(ex, emul)
    log(f"  vs emulation max err {maxerr:.3e} (tol {tol:.3e}); vs exact gpu {m_gpu} emul {m_em}")
    assert m_gpu["cos"] >= min(0.999, m_em["cos"] - 2e-4)
    assert m_gpu["rel_l1"] <= max(0.02, m_em["rel_l1"] + 0.003)
    return gpu


SMALL = {
    "tiny": ("tiny", {}),
    "tiny_causal": ("tiny", {"causal": True}),
    "llm_prefill_ragged": ("llm_prefill", dict(B=1, H=2, N=1000)),
    "image_dit_int4": ("image_dit", dict(B=1, H=2, N=777)),
    "video_dit_tail": ("video_dit", dict(H=2, N=1500)),
    "long_context_int8": ("long_context", dict(H=2, N=900)),
    "long_context_int4": ("long_context_int4", dict(H=2, N=900)),
    "target_small": ("target", dict(H=2, N=640)),
    "target_causal_small": ("target_causal", dict(H=2, N=700)),
    "d64_bf16": ("tiny", dict(dtype="bf16", N=300, H=3)),
    "d128_fp16": ("target", dict(dtype="fp16", H=2, N=513)),
    "batch2": ("llm_prefill", dict(B=2, H=3, N=260)),
    "n1": ("tiny", dict(N=1)),
    "n127": ("tiny", dict(N=127)),
    "n129_causal": ("tiny", dict(N=129, causal=True)),
    "n255_d128": ("target", dict(H=1, N=255)),
    "one_head_n9000": ("target", dict(H=1, N=9000)),            # 71 blocks: batched finalize path
    "one_head_n9000_causal_int4": ("long_context_int4", dict(H=1, N=9000)),
}


@pytest.mark.parametrize("case", sorted(SMALL))
def test_parity(case):
    name, over = SMALL[case]
    _check_case(scaled(WORKLOADS[name], **over))


def _degenerate(kind, causal):
    w = scaled(WORKLOADS["target_causal" if causal else "target"], H=2, N=300)
    q, k, v = make_inputs(w)
    if kind == "constant_k":        # every key of a head equals its first: K' = 0, all K codes 0
        k[:] = k[:, :, :1, :]
    elif kind == "zero_q_block":    # query block 1 all zero: its mean and codes are 0
        q[:, :, 128:256, :] = 0.0
    elif kind == "constant_v":      # V' = 0: every channel's range is 0
        v[:] = v[:, :, :1, :]
    elif kind == "all_zero":
        q[:], k[:], v[:] = 0.0, 0.0, 0.0
    elif kind == "outliers":        # single large values (exact in bf16) in Q, K and V
        q[0, 0, 5, 3], k[0, 1, 17, 40], v[0, 1, 250, 7] = 96.0, -80.0, 120.0
    return w, q, k, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["constant_k", "zero_q_block", "constant_v", "all_zero", "outliers"])
def test_degenerate_inputs(kind, causal):
    """Inputs whose groups have zero range, or single outliers: codes, scales and
    means stay bit-exact and the output meets the same bars; where the output
    has a closed form (V constant over tokens, everything zero) it is exact."""
    w, q, k, v = _degenerate(kind, causal)
    gpu = _check_inputs(w, q, k, v, vs_exact=kind not in ("constant_v", "all_zero"))
    if kind in ("constant_v", "all_zero"):
        # O = sum P~ V' / l + mean(V) with V' = 0: every row is V's (dtype-exact) token row
        want = np.broadcast_to(v[:, :, :1, :], v.shape)
        np.testing.assert_array_equal(gpu["out"], want)


@pytest.mark.parametrize("gran", ["warp", "block"])
@pytest.mark.parametrize("bits", [8, 4])
def test_granularities(gran, bits):
    _check_case(scaled(WORKLOADS["llm_prefill"], B=1, H=2, N=600, qk_bits=bits), gran=gran)


@pytest.mark.parametrize("smooth", [(False, False, False), (True, False, True), (False, True, False)])
def test_smoothing_flags(smooth):
    _check_case(scaled(WORKLOADS["image_dit"], B=1, H=2, N=400, qk_bits=8), smooth=smooth)


def test_sa2pp_ranges():
    # SageAttention2++ summary, 3.1: P_r = 224 and V_r = 4.5.
    _check_case(scaled(WORKLOADS["video_dit"], H=2, N=700), p_range=224.0, v_range=4.5)


def test_strided_inputs():
    _check_case(scaled(WORKLOADS["llm_prefill"], B=2, H=2, N=333), layout="bnhd")


def test_widest_row_stride():
    # rows 2^22 - 8 elements apart (8 MiB each): the quantisers' 32-bit buffer
    # offsets at their largest, with a ragged last block (130 = 128 + 2 rows)
    _check_case(scaled(WORKLOADS["target"], B=1, H=1, N=130), layout="widest_rows")


def test_repeatable_bits():
    w = scaled(WORKLOADS["target"], H=2, N=900)
    q, k, v = make_inputs(w)
    a = run_sage(q, k, v, w.dtype, w.causal, w.qk_bits, w.gran)
    b = run_sage(q, k, v, w.dtype, w.causal, w.qk_bits, w.gran)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)


def test_one_shot_call_matches_three_calls():
    import torch
    from quantized_attention_sage_amd import api
    from gpu_harness import to_device
    w = scaled(WORKLOADS["llm_prefill"], B=1, H=2, N=500)
    q, k, v = make_inputs(w)
    three = run_sage(q, k, v, w.dtype, w.causal, w.qk_bits, w.gran, download=())
    qt, kt, vt = (to_device(x, w.dtype) for x in (q, k, v))
    o = api.attn(qt, kt, vt, causal=w.causal, qk_bits=w.qk_bits, gran=w.gran)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o.float().cpu().numpy(), three["out"])


def test_invalid_arguments_launch_nothing():
    import torch
    from quantized_attention_sage_amd import api, SageError
    x = torch.zeros(1, 1, 64, 96, dtype=torch.bfloat16, device="cuda")      # d = 96 unsupported
    with pytest.raises(SageError):
        api.attn(x, x, x)
    y = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(y, 7.0)
    with pytest.raises(SageError):
        api.attn(y, y, y, out=out, p_range=500.0)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
