"""A whole step captured in a HIP graph.

The entry points allocate nothing and enqueue no memset (only kernels on the
caller's stream), so serving loops can capture quant_qk + quant_v + attn_fwd
once and replay them.  Every replay must equal the eager result bit for bit,
with eager work and synchronisations between replays, and a replay after the
inputs change in place must equal the eager step on the new inputs.
"""
import pytest

from quantized_attention_sage_amd.workloads import WORKLOADS, scaled, make_inputs
from gpu_harness import to_device, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("qk_format,pv", [("int", "fp8"), ("mxfp4", "fp8"), ("int", "f16"), ("int_e2m3", "fp8")])
def test_graph_replay_matches_eager(qk_format, pv):
    import torch
    from quantized_attention_sage_amd import api

    w = scaled(WORKLOADS["target_causal"], H=2, N=900)
    log(f"graph case qk={qk_format} pv={pv}: H={w.H} N={w.N} causal={w.causal}")
    q, k, v = make_inputs(w)
    qt, kt, vt = (to_device(x, w.dtype) for x in (q, k, v))
    bits = 4 if qk_format.startswith("int_") else w.qk_bits     # the held formats carry INT4-range codes
    params = api.make_params(qk_bits=bits, gran=w.gran, qk_format=qk_format, pv=pv)
    shape = api.make_shape(qt, kt, vt)
    ws = api.Workspace(shape, params, qt.device)
    out = torch.empty_like(qt)

    def step():
        api.quant_qk(qt, kt, vt, params, ws, shape)
        api.quant_v(vt, params, ws, shape)
        api.attn_fwd(ws, shape, params, w.causal, out)

    step()
    torch.cuda.synchronize()
    ref = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    for r in range(4):
        out.zero_()
        ws.tensor.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs from the eager step"

    vt.mul_(2)                       # exact in bf16/fp16: the replay must read the new V
    g.replay()
    torch.cuda.synchronize()
    replayed = out.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(replayed, out)
    assert not torch.equal(replayed, ref)


@pytest.mark.parametrize("causal", [False, True])
def test_training_step_graph_replay_matches_eager(causal):
    """The 8-bit training step (both quantisation calls, the forward with L and
    the backward, whose operand passes reuse the quantisation kernels) captured
    once: every replay equals the eager O, L and gradients bit for bit, and a
    replay after dO changes in place equals the eager step on the new dO."""
    import torch
    from quantized_attention_sage_amd import api
    from quantized_attention_sage_amd.workloads import make_grad

    w = scaled(WORKLOADS["target_causal" if causal else "target"], H=2, N=700)
    log(f"training-step graph case: H={w.H} N={w.N} causal={causal}")
    q, k, v = make_inputs(w)
    qt, kt, vt = (to_device(x, w.dtype) for x in (q, k, v))
    params = api.make_params(qk_bits=8, gran="thread")   # the backward's setting
    shape = api.make_shape(qt, kt, vt)
    ws = api.Workspace(shape, params, qt.device)
    bws = api.BwdWorkspace(shape, params, qt.device)
    out = torch.empty_like(qt)
    do = to_device(make_grad(w), w.dtype)
    lse = torch.empty((w.B, w.H, ws.layout.n_pad), dtype=torch.float32, device=qt.device)
    grads = [torch.empty(qt.shape, dtype=torch.float32, device=qt.device) for _ in range(3)]

    def step():
        api.quant_qk(qt, kt, vt, params, ws, shape)
        api.quant_v(vt, params, ws, shape)
        api.attn_fwd_lse(ws, shape, params, causal, out, lse)
        api.attn_bwd(qt, kt, vt, out, do, lse, ws, shape, params, causal, bws, *grads)

    def results():
        return [out.clone(), lse.clone()] + [g_.clone() for g_ in grads]

    def clear():
        for t_ in [out, lse, ws.tensor, bws.tensor] + grads:
            t_.zero_()

    step()
    torch.cuda.synchronize()
    ref = results()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    names = ("O", "L", "dQ", "dK", "dV")
    for r in range(3):
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(names, results(), ref):
            assert torch.equal(a, b), f"replay {r}: {n} differs from the eager step"

    do.mul_(2)                       # exact: the replay must read the new dO
    g.replay()
    torch.cuda.synchronize()
    replayed = results()
    step()
    torch.cuda.synchronize()
    for n, a, b in zip(names, replayed, results()):
        assert torch.equal(a, b), f"{n}: the replay after dO changed differs from the eager step"
    assert not torch.equal(replayed[4], ref[4])
