"""sage_attn_static: the one-shot call with every intermediate in the
library-held static workspace, against sage_attn with a caller workspace.

Both run the same kernels on the same inputs, so the outputs must agree bit
for bit.  Two calls in a row (the second smaller, on another stream) check
that nothing left in the shared array from the first call leaks into the
second."""
import numpy as np
import pytest

from quantized_attention_sage_amd.workloads import WORKLOADS, make_inputs, scaled
from gpu_harness import to_device, log, GuardedOut

pytestmark = pytest.mark.gpu


def _pair(w, stream=None):
    import torch
    from quantized_attention_sage_amd import api
    q, k, v = make_inputs(w)
    qt, kt, vt = (to_device(x, w.dtype) for x in (q, k, v))
    kw = dict(qk_bits=w.qk_bits, gran=w.gran)
    ref = api.attn(qt, kt, vt, causal=w.causal, **kw)
    g = GuardedOut(qt)
    if stream is None:
        api.attn_static(qt, kt, vt, causal=w.causal, out=g.out, **kw)
    else:
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            api.attn_static(qt, kt, vt, causal=w.causal, out=g.out, **kw)
        torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g.check()
    return ref.float().cpu().numpy(), g.out.float().cpu().numpy()


def test_static_workspace_matches_caller_workspace_twice():
    import torch
    first = scaled(WORKLOADS["target"], H=4, N=1000)
    second = scaled(WORKLOADS["llm_prefill"], B=1, H=2, N=300)      # smaller, causal
    for i, (w, stream) in enumerate(((first, None), (second, torch.cuda.Stream()))):
        log(f"static-workspace call {i}: {w.name} B={w.B} H={w.H} N={w.N} causal={w.causal}")
        ref, got = _pair(w, stream)
        np.testing.assert_array_equal(got, ref, err_msg=f"call {i}")


def test_static_workspace_rejects_a_problem_that_does_not_fit():
    import torch
    from quantized_attention_sage_amd import api, SageError
    from quantized_attention_sage_amd import _lib as L
    x = torch.zeros(1, 16, 8192, 128, dtype=torch.bfloat16, device="cuda")   # needs about 80 MiB
    out = torch.full_like(x, 3.0)
    with pytest.raises(SageError) as e:
        api.attn_static(x, x, x, out=out)
    assert e.value.status == L.SAGE_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
