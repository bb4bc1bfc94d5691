"""GPU parity of the 8-bit training path: sage_attn_fwd_lse and sage_attn_bwd
against the CPU oracle (oracle/backward.py).

The backward takes O and L from the oracle's own emulated forward (uploaded),
so both sides differentiate the same forward; the GPU forward's L is checked
separately.  Bars:
  * the backward's INT8 dO / V codes and scales, its E4M3 dO, Q and K' codes
    and scales: bit-exact (the same quantisers as the forward's, already
    bit-exact);
  * D: within 4 ulp-scale relative error (fp32 sums in another order);
  * L of the forward: within 2^-18 (1 + |L|) (fp32 exp2 / log2 of the kernel);
  * dQ, dK, dV against the emulation: sum |G - E| <= 5e-4 sum |E|, and
    elementwise |G - E| <= 1e-2 max|E|.  The two sides accumulate in another
    order (about 1e-6 relative) and, rarely, decide an E4M3 code of P or dS
    from fp32 values that differ in their last bits (exp2 and the order of
    the fp32 products); such a flip moves one product term of one element by
    one E4M3 step, at most 2^-3 of that term.  A wrong axis, scale, mask or
    operand moves every element and fails the sum bar by orders of magnitude;
  * against exact float64 gradients: the GPU's cosine and relative L1 equal
    the emulation's within 1e-4 and 5e-4 (the accuracy is the method's).
"""
import numpy as np
import pytest

import oracle
from oracle import backward as ob
from quantized_attention_sage_amd.workloads import WORKLOADS, make_grad, make_inputs, scaled
from gpu_harness import CANARY, GUARD, _check_canary, _guard_regions, log, to_device, unpermute_v

pytestmark = pytest.mark.gpu

CASES = {
    "target_small": ("target", dict(H=2, N=640)),
    "target_causal_small": ("target_causal", dict(H=2, N=700)),
    "llm_prefill_ragged_causal": ("llm_prefill", dict(B=1, H=2, N=300)),
    "image_dit": ("image_dit", dict(B=1, H=2, N=400, qk_bits=8)),
    "d64_fp16_tiny": ("tiny", dict(N=300)),
    "d64_fp16_causal": ("tiny", dict(N=200, causal=True)),
    "batch2": ("video_dit", dict(B=2, H=2, N=260)),
    "n1": ("tiny", dict(N=1)),
    "long_context_one_head": ("long_context", dict(H=1, N=1100)),
}


def _guarded_bwd_workspace(shape, params, device):
    import ctypes
    import torch
    from quantized_attention_sage_amd import api, _lib as L

    class GuardedBwd(api.BwdWorkspace):
        def __init__(self):
            lay = L.BwdLayout()
            L.check(L.lib().sage_bwd_workspace_layout(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(lay)))
            self.layout = lay
            self.shape = (shape.B, shape.H, shape.N, shape.d)
            self.tensor = torch.full((lay.total_bytes + 2 * GUARD + 256,), CANARY, dtype=torch.uint8, device=device)
            self._pad = (-self.tensor.data_ptr()) % 256 + GUARD

        def check_guards(self):
            spans = [(getattr(self.layout, n).offset, getattr(self.layout, n).bytes) for n in L.BWD_SPANS]
            _check_canary(self.tensor, _guard_regions(spans, self._pad, self.layout.total_bytes,
                                                      self.tensor.numel()), "backward workspace")

    return GuardedBwd()


class _GuardedF32:
    """fp32 tensor shaped like `like` between two canary bands."""

    def __init__(self, like):
        import torch
        n, self.g = like.numel(), GUARD // 4
        self.buf = torch.full((n + 2 * self.g,), float("nan"), dtype=torch.float32, device=like.device)
        self.buf[:self.g] = 12345.0
        self.buf[-self.g:] = 12345.0
        self.t = self.buf[self.g:self.g + n].view(like.shape)

    def check(self, what):
        assert bool((self.buf[:self.g] == 12345.0).all()) and bool((self.buf[-self.g:] == 12345.0).all()), what


def run_backward(w):
    import torch
    from quantized_attention_sage_amd import api
    from gpu_harness import guarded_workspace, GuardedOut
    q, k, v = make_inputs(w)
    do = make_grad(w)
    o_em, lse_em, qk_o, vq_o = ob.forward_with_lse(q, k, v, w.causal, w.dtype)

    qt, kt, vt, dot = (to_device(x, w.dtype) for x in (q, k, v, do))
    params = api.make_params(qk_bits=8, gran="thread")
    shape = api.make_shape(qt, kt, vt)
    ws = guarded_workspace(shape, params, qt.device)
    api.quant_qk(qt, kt, vt, params, ws, shape)
    api.quant_v(vt, params, ws, shape)
    g = GuardedOut(qt)
    lse_gpu = torch.full((w.B, w.H, ws.layout.n_pad), float("nan"), dtype=torch.float32, device=qt.device)
    api.attn_fwd_lse(ws, shape, params, w.causal, g.out, lse_gpu)

    ot = to_device(o_em, w.dtype)
    lse_t = torch.from_numpy(lse_em).cuda()
    bws = _guarded_bwd_workspace(shape, params, qt.device)
    grads = [_GuardedF32(qt) for _ in range(3)]
    api.attn_bwd(qt, kt, vt, ot, dot, lse_t, ws, shape, params, w.causal, bws, *(x.t for x in grads))
    torch.cuda.synchronize()
    ws.check_guards()
    g.check()
    bws.check_guards()
    for x, n in zip(grads, ("dq", "dk", "dv")):
        x.check(n)
    gpu = {n: bws.view(n).cpu().numpy() for n in ("do_codes", "do_scale", "v_codes", "v_scale", "do8_codes",
                                                   "do8_scale", "q8_codes", "q8_scale", "k8_codes", "k8_scale",
                                                   "dsum", "lse_do", "dsum_do")}
    return dict(q=q, k=k, v=v, do=do, o_em=o_em, lse_em=lse_em, qk_o=qk_o, vq_o=vq_o,
                fwd_codes=(ws.view("q_codes").cpu().numpy(), ws.view("k_codes").cpu().numpy()),
                lse_gpu=lse_gpu.cpu().numpy(), ops=gpu, grads=[x.t.cpu().numpy().astype(np.float64) for x in grads])


def _bits(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_parity(case):
    name, over = CASES[case]
    w = scaled(WORKLOADS[name], **over)
    log(f"backward case {case}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    r = run_backward(w)
    np.testing.assert_array_equal(r["fwd_codes"][0], r["qk_o"]["q_codes"])
    np.testing.assert_array_equal(r["fwd_codes"][1], r["qk_o"]["k_codes"])

    # the forward's L
    n_rows = w.N
    dl = np.abs(r["lse_gpu"][:, :, :n_rows] - r["lse_em"][:, :, :n_rows])
    assert np.all(dl <= 2.0 ** -18 * (1 + np.abs(r["lse_em"][:, :, :n_rows]))), float(dl.max())

    ctx = ob.prepare(r["q"], r["k"], r["v"], r["do"], r["o_em"], r["lse_em"], r["qk_o"], w.causal)
    ops = r["ops"]
    dov = ctx["dov"]
    np.testing.assert_array_equal(ops["do_codes"], dov["q_codes"], err_msg="INT8 dO codes")
    np.testing.assert_array_equal(_bits(ops["do_scale"]), _bits(dov["q_scale"]), err_msg="INT8 dO scales")
    np.testing.assert_array_equal(ops["v_codes"], dov["k_codes"], err_msg="INT8 V codes")
    np.testing.assert_array_equal(_bits(ops["v_scale"]), _bits(dov["k_scale"]), err_msg="INT8 V scales")
    for n in ("do", "q", "k"):
        np.testing.assert_array_equal(unpermute_v(ops[f"{n}8_codes"]), ctx["fp8"][n]["v_codes"], err_msg=f"E4M3 {n}")
        np.testing.assert_array_equal(_bits(ops[f"{n}8_scale"]), _bits(ctx["fp8"][n]["v_scale"]),
                                      err_msg=f"E4M3 {n} scales")
    dd = np.abs(ops["dsum"].astype(np.float64) - ctx["D"])
    d_tol = 1e-6 * (np.abs(ctx["D"]) + np.abs(r["do"]).max() * np.abs(r["o_em"]).max())
    assert np.all(dd <= d_tol), float(dd.max())
    # the dK kernel's per-row terms L - log2 s and D / s (s: the row's INT8 dO
    # scale), from the oracle's L, D and scales; +inf and 0 where s = 0
    s_do = dov["q_scale"].astype(np.float64)[:, :, :n_rows]
    pos = s_do > 0
    lse_do, dsum_do = ops["lse_do"][:, :, :n_rows], ops["dsum_do"][:, :, :n_rows]
    want_l = r["lse_em"][:, :, :n_rows].astype(np.float64) - np.log2(np.where(pos, s_do, 1.0))
    want_d = ctx["D"][:, :, :n_rows] / np.where(pos, s_do, 1.0)
    assert np.all(np.abs(lse_do[pos] - want_l[pos]) <= 2.0 ** -20 * (1 + np.abs(want_l[pos])))
    assert np.all(np.abs(dsum_do[pos] - want_d[pos]) <= d_tol[:, :, :n_rows][pos] / s_do[pos] + 2.0 ** -22 * np.abs(want_d[pos]))
    assert np.all(np.isposinf(lse_do[~pos])) and np.all(dsum_do[~pos] == 0)

    em = ob.emulate_backward(ctx)
    ex = ob.exact_attention_grad(r["q"], r["k"], r["v"], r["do"], w.causal)
    for nm, gg, ee, xx in zip(("dQ", "dK", "dV"), r["grads"], em, ex):
        err = np.abs(gg - ee)
        scale = np.abs(ee).max()
        # N = 1: dQ = dK = 0 exactly, and the metrics against exact gradients are undefined
        defined = np.abs(xx).max() > 1e-12
        m_g, m_e = (oracle.compare(xx, gg), oracle.compare(xx, ee)) if defined else ({}, {})
        vs_exact = (f"vs exact gpu cos {m_g['cos']:.6f} relL1 {m_g['rel_l1']:.4f}, emul cos {m_e['cos']:.6f} "
                    f"relL1 {m_e['rel_l1']:.4f}") if defined else "exact gradient is zero"
        log(f"  {nm}: max|gpu - emul| = {err.max():.3e} ({err.max() / max(scale, 1e-30):.2e} of max|G|), "
            f"rel L1 {err.sum() / max(np.abs(ee).sum(), 1e-30):.2e}; {vs_exact}")
        assert err.sum() <= 5e-4 * np.abs(ee).sum() + 1e-30, f"{nm}: sum |G - E| / sum |E| too large"
        assert np.all(err <= 1e-2 * scale + 1e-30), f"{nm}: {int((err > 1e-2 * scale).sum())} elements beyond 1e-2 max|E|"
        if defined:
            assert abs(m_g["cos"] - m_e["cos"]) <= 1e-4 and abs(m_g["rel_l1"] - m_e["rel_l1"]) <= 5e-4


def _sample(n):
    return sorted({0, n // 2, n - 1})


@pytest.mark.parametrize("name", ["target", "target_causal"])
def test_backward_fullsize_sampled(name):
    """The target shape (B=1, H=32, N=16384, d=128) in the launch configuration
    bench.py --backward times.  One head's O and L come from the oracle's
    forward (the others from the GPU's); its sampled query blocks (dQ) and key
    blocks (dK, dV) are checked against the emulation with the bars above."""
    import torch
    from quantized_attention_sage_amd import api
    from oracle.quant import QuantParams
    w = WORKLOADS[name]
    log(f"full-size backward case {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    q, k, v = make_inputs(w)
    do = make_grad(w)
    b, h = 0, w.H // 2
    sl = (slice(b, b + 1), slice(h, h + 1))
    qh, kh, vh, doh = (x[sl] for x in (q, k, v, do))
    o_em, lse_em, qk1, _ = ob.forward_with_lse(qh, kh, vh, w.causal, w.dtype, QuantParams())
    log("  oracle forward of the checked head done")

    qt, kt, vt, dot = (to_device(x, w.dtype) for x in (q, k, v, do))
    params = api.make_params(qk_bits=8, gran="thread")
    shape = api.make_shape(qt, kt, vt)
    ws = api.Workspace(shape, params, qt.device)
    out = torch.empty_like(qt)
    lse = torch.empty((w.B, w.H, ws.layout.n_pad), dtype=torch.float32, device=qt.device)
    api.quant_qk(qt, kt, vt, params, ws, shape)
    api.quant_v(vt, params, ws, shape)
    api.attn_fwd_lse(ws, shape, params, w.causal, out, lse)
    out[b, h] = torch.from_numpy(o_em[0, 0]).to(out.dtype).cuda()
    lse[b, h] = torch.from_numpy(lse_em[0, 0]).cuda()
    bws = api.BwdWorkspace(shape, params, qt.device)
    grads = [torch.empty(qt.shape, dtype=torch.float32, device=qt.device) for _ in range(3)]
    api.attn_bwd(qt, kt, vt, out, dot, lse, ws, shape, params, w.causal, bws, *grads)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ws.view("q_codes")[b, h].cpu().numpy(), qk1["q_codes"][0, 0])
    g = [x[b, h].cpu().numpy().astype(np.float64) for x in grads]
    del grads, qt, kt, vt, dot, out, ws, bws

    ctx = ob.prepare(qh, kh, vh, doh, o_em, lse_em, qk1, w.causal)
    nblk = qk1["n_pad"] // 128
    for blk in _sample(nblk):
        rows = slice(128 * blk, min(w.N, 128 * blk + 128))
        n = rows.stop - rows.start
        want = [ob.dq_block(ctx, 0, 0, blk)[:n], *(x[:n] for x in ob.dkdv_block(ctx, 0, 0, blk))]
        for nm, gg, ee in zip(("dQ", "dK", "dV"), (g[0][rows], g[1][rows], g[2][rows]), want):
            err = np.abs(gg - ee)
            log(f"  block {blk} {nm}: sum|G - E| / sum|E| = {err.sum() / np.abs(ee).sum():.2e}, "
                f"max {err.max() / np.abs(ee).max():.2e} of max|E|")
            assert err.sum() <= 5e-4 * np.abs(ee).sum(), (blk, nm)
            assert np.all(err <= 1e-2 * np.abs(ee).max()), (blk, nm)
