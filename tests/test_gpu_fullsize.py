"""GPU parity at the full benchmark sizes, on sampled heads and query blocks.

Every workload recipe runs at its full size through the same entry points and
launch configuration bench.py times (default parameters, one workspace).  The
oracle is independent per head, so for a few sampled heads it recomputes the
codes, scales and means (compared bit for bit), the bias (within the split
bf16 bound) and the emulated output of sampled 128-query blocks (within
2e-3 max|V| plus half an output ulp), plus exact fp64 attention on those rows
(the GPU must be as accurate as the emulation of the method).  Bars as in
test_gpu_parity.py.
"""
import numpy as np
import pytest

import oracle
from oracle.attention import emulate_block, exact_attention_rows
from oracle.quant import QuantParams
from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs
from gpu_harness import (assert_quant_bit_exact, bias_tolerance_ok, output_tolerance, to_device, log, BUFFERS,
                         unpermute_v, guarded_workspace, GuardedOut)

pytestmark = pytest.mark.gpu

FULL = ["llm_prefill", "image_dit", "video_dit", "long_context", "long_context_int4", "target", "target_causal"]
# the other Q/K and P~V formats at the target shape, and the E4M3-held INT4-range
# codes on the INT4-range recipes: (recipe, qk_format, pv)
MODES = [("target", "mxfp4", "fp8"), ("target_causal", "mxfp4", "fp8"), ("target", "int", "f16"),
         ("long_context_int4", "int_e4m3", "fp8"), ("image_dit", "int_e4m3", "fp8"),
         ("long_context_int4", "int_e2m3", "fp8"), ("image_dit", "int_e2m3", "fp8")]


# (recipe, qk_format) whose middle head is compared block by block in full: every
# query block against the emulation, every row against exact attention
FULL_HEAD = {("target", "int"), ("target_causal", "int"), ("target", "mxfp4"), ("target_causal", "mxfp4")}
# the accuracy bar against exact attention named for the method (cos >= 0.999,
# rel L1 <= 0.02); reported per recipe, asserted only relative to the emulation
NS_COS, NS_RL1 = 0.999, 0.02


def _heads(w):
    return sorted({(0, 0), (w.B // 2, w.H // 2), (w.B - 1, w.H - 1)})


def _blocks(n_blocks):
    return sorted({0, n_blocks // 2, n_blocks - 1})


def _metrics(ref, x):
    ref = ref.astype(np.float64).ravel()
    x = x.astype(np.float64).ravel()
    return float(ref @ x / (np.linalg.norm(ref) * np.linalg.norm(x))), float(np.abs(ref - x).sum() / np.abs(ref).sum())


@pytest.mark.parametrize("name", FULL)
def test_fullsize_sampled(name):
    _fullsize(name, "int", "fp8")


@pytest.mark.parametrize("name,qk_format,pv", MODES)
def test_fullsize_sampled_formats(name, qk_format, pv):
    _fullsize(name, qk_format, pv)


def _fullsize(name, qk_format, pv):
    import torch
    from quantized_attention_sage_amd import api
    from gpu_harness import unpermute_v16, half_bits

    w = WORKLOADS[name]
    log(f"full-size case {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} bits={w.qk_bits} "
        f"qk={qk_format} pv={pv}")
    q, k, v = make_inputs(w)
    vmax = float(np.abs(v).max())
    qt, kt, vt = (to_device(x, w.dtype) for x in (q, k, v))
    params = api.make_params(qk_bits=w.qk_bits, gran=w.gran, qk_format=qk_format, pv=pv)
    shape = api.make_shape(qt, kt, vt)
    ws = guarded_workspace(shape, params, qt.device)
    g = GuardedOut(qt)
    out = g.out
    api.quant_qk(qt, kt, vt, params, ws, shape)
    api.quant_v(vt, params, ws, shape)
    api.attn_fwd(ws, shape, params, w.causal, out)
    torch.cuda.synchronize()
    ws.check_guards()
    g.check()
    del qt, kt, vt

    p = QuantParams(qk_bits=w.qk_bits, gran=w.gran, qk_format=qk_format, pv=w.dtype if pv == "f16" else "fp8")
    ex_all, gpu_all, em_all = [], [], []
    for (b, h) in _heads(w):
        qh, kh, vh = (x[b:b + 1, h:h + 1] for x in (q, k, v))
        qk1 = oracle.quant_qk(qh, kh, p)
        vq1 = oracle.quant_v(vh, p)
        gpu = {n: ws.view(n)[b:b + 1, h:h + 1].cpu().numpy() for n in BUFFERS}
        if qk_format == "int" and pv == "fp8":
            assert_quant_bit_exact(gpu, qk1, vq1)
        else:
            for n in ("q_codes", "k_codes", "q_scale", "k_scale", "q_mean", "k_mean"):
                np.testing.assert_array_equal(gpu[n].view(np.uint8), qk1[n].view(np.uint8), err_msg=n)
            if pv == "f16":
                np.testing.assert_array_equal(unpermute_v16(gpu["v_codes"]), half_bits(vq1["v_values"], w.dtype))
            else:
                np.testing.assert_array_equal(unpermute_v(gpu["v_codes"]), vq1["v_codes"], err_msg="v codes")
        ok, worst = bias_tolerance_ok(gpu["bias"], qk1["bias"], qk1["q_mean"], qk1["k_smoothed"])
        assert ok, f"head {(b, h)}: bias error {worst} of the bound"
        o_gpu = out[b, h].float().cpu().numpy()
        full_head = (name, qk_format) in FULL_HEAD and pv == "fp8" and (b, h) == (w.B // 2, w.H // 2)
        for qb in (range(qk1["n_pad"] // 128) if full_head else _blocks(qk1["n_pad"] // 128)):
            em, rows = emulate_block(qk1, vq1, 0, 0, qb, w.causal)
            g = o_gpu[rows]
            tol = output_tolerance(vh, em, w.dtype) - 2e-3 * float(np.abs(vh).max()) + 2e-3 * vmax
            bad = np.abs(g - em) > tol
            assert not bad.any(), (f"head {(b, h)} block {qb}: {int(bad.sum())} outputs beyond tolerance, "
                                   f"max err {float(np.abs(g - em).max())}")
            ex = exact_attention_rows(qh[0, 0], kh[0, 0], vh[0, 0], rows, w.causal)
            ex_all.append(ex)
            gpu_all.append(g)
            em_all.append(em)
        log(f"  head {(b, h)}: codes/scales/means bit-exact, bias within bound, "
            f"{'every' if full_head else 'sampled'} query block within tolerance")
    ex_all, gpu_all, em_all = (np.concatenate(x) for x in (ex_all, gpu_all, em_all))
    cos_g, rl1_g = _metrics(ex_all, gpu_all)
    cos_e, rl1_e = _metrics(ex_all, em_all)
    log(f"  vs exact on sampled rows: gpu cos {cos_g:.6f} relL1 {rl1_g:.4f}; emulation cos {cos_e:.6f} relL1 {rl1_e:.4f}")
    met = cos_g >= NS_COS and rl1_g <= NS_RL1
    log(f"  ACCURACY {name} qk={qk_format} pv={pv}: cos {cos_g:.6f} relL1 {rl1_g:.4f} against the bar "
        f"cos >= {NS_COS}, relL1 <= {NS_RL1}: {'met' if met else 'NOT met'}"
        f"{'' if met else ' (the emulation of the method gets cos %.6f relL1 %.4f)' % (cos_e, rl1_e)}")
    assert cos_g >= min(0.999, cos_e - 2e-4)
    assert rl1_g <= max(0.02, rl1_e + 0.003)
