"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle.  Inputs come from the shared seeded generators; no
expected value comes from the HIP path."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from oracle.attention import round_output

BUFFERS = ("q_codes", "q_scale", "q_mean", "k_codes", "k_scale", "k_mean", "bias",
           "v_codes", "v_scale", "v_mean")


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16}[name]


def to_device(x: np.ndarray, dtype: str, layout: str = "bhnd"):
    """Upload exactly-representable float32 values as fp16/bf16.

    layout "bnhd" stores the tensor as [B, N, H, d] and returns the
    [B, H, N, d] view (non-contiguous strides through the ABI); "widest_rows"
    puts consecutive tokens WIDEST_ROW_STRIDE elements apart (the largest N
    stride the library accepts), the rest of each row zero.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype))
    if layout == "bnhd":
        t = t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    elif layout == "widest_rows":
        B, H, N, d = t.shape
        wide = torch.zeros((B, H, N, WIDEST_ROW_STRIDE), dtype=t.dtype, device="cuda")
        wide[..., :d] = t.cuda()
        t = wide[..., :d]
    else:
        t = t.cuda()
    return t


# the largest N stride (elements) the library accepts: below 2^22, a multiple of 8
WIDEST_ROW_STRIDE = (1 << 22) - 8


# ------------------------------------------------------------------ guard bands
# Canary bytes before, between and after every span the library may write; a
# kernel that writes outside its buffer changes one of them.
GUARD = 4096          # bytes of canary before the first and after the last span
CANARY = 0xA5
OUT_CANARY = 0x7FA5   # 16-bit canary around outputs (a NaN pattern in fp16 and bf16)


def _guard_regions(spans, base, total, length):
    """[lo, hi) byte ranges of a guarded allocation that no span covers."""
    regions, pos = [(0, base)], base
    for off, size in sorted(spans):
        if base + off > pos:
            regions.append((pos, base + off))
        pos = max(pos, base + off + size)
    regions.append((max(pos, base + total), length))
    return [(lo, hi) for lo, hi in regions if hi > lo]


def _check_canary(t, regions, what):
    for lo, hi in regions:
        bad = int((t[lo:hi] != CANARY).sum().item())
        assert bad == 0, f"{what}: {bad} canary bytes overwritten in [{lo}, {hi})"


def guarded_workspace(shape, params, device):
    """A Workspace whose allocation is pre-filled with canary bytes and has a
    guard band before and after; .check_guards() verifies every byte outside
    the spans of sage_layout is untouched."""
    import ctypes
    import torch
    from quantized_attention_sage_amd import api, _lib as L

    class GuardedWorkspace(api.Workspace):
        def __init__(self):
            lay = L.Layout()
            L.check(L.lib().sage_workspace_layout(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(lay)))
            self.layout = lay
            self.shape = (shape.B, shape.H, shape.N, shape.d)
            self.pv_f16 = params.pv_mode == L.PV_MODE["f16"]
            self.qk_mx = params.qk_format == L.QK_FORMAT["mxfp4"]
            self.qk_held = params.qk_format in (L.QK_FORMAT["int_e4m3"], L.QK_FORMAT["int_e2m3"])
            self.tensor = torch.full((lay.total_bytes + 2 * GUARD + 256,), CANARY, dtype=torch.uint8, device=device)
            self._pad = (-self.tensor.data_ptr()) % 256 + GUARD
            self.qk = L.QKBuffers()
            self.vb = L.VBuffers()
            L.check(L.lib().sage_bind_workspace(ctypes.byref(lay), ctypes.c_void_p(self.ptr),
                                                ctypes.c_size_t(lay.total_bytes), ctypes.byref(self.qk),
                                                ctypes.byref(self.vb)))

        def check_guards(self):
            lay = self.layout
            names = ("q_codes", "q_scale", "q_mean", "k_codes", "k_scale", "k_mean", "bias", "k_partial",
                     "v_codes", "v_scale", "v_mean", "v_partial")
            spans = [(getattr(lay, n).offset, getattr(lay, n).bytes) for n in names]
            _check_canary(self.tensor, _guard_regions(spans, self._pad, lay.total_bytes, self.tensor.numel()),
                          "workspace")

    return GuardedWorkspace()


class GuardedOut:
    """An output tensor shaped like `like` (contiguous [B,H,N,d]) inside a larger
    allocation whose ends hold a 16-bit canary."""

    def __init__(self, like, guard_elems=GUARD // 2):
        import torch
        n = like.numel()
        self.g = guard_elems
        self.buf = torch.full((n + 2 * guard_elems,), OUT_CANARY, dtype=torch.int16, device=like.device)
        self.out = self.buf[guard_elems:guard_elems + n].view(like.dtype).view(like.shape)

    def check(self):
        for part in (self.buf[:self.g], self.buf[-self.g:]):
            bad = int((part != OUT_CANARY).sum().item())
            assert bad == 0, f"output guard: {bad} canary elements overwritten"


def guarded_probe_scratch(shape, device):
    """A ProbeScratch pre-filled with canary bytes, with a guard band before and
    after, and canaries in the alignment gaps between its three row spans
    (exact fp32 rows, INT4-range rows, INT8 rows, each [B, H, 128, d]).
    .check_guards() verifies them; rows past N inside a span are unspecified."""
    import ctypes
    import torch
    from quantized_attention_sage_amd import api, _lib as L

    class GuardedProbeScratch(api.ProbeScratch):
        def __init__(self):
            n = ctypes.c_size_t()
            L.check(L.lib().sage_probe_scratch_bytes(ctypes.byref(shape), ctypes.byref(n)))
            self.nbytes = n.value
            self.tensor = torch.full((self.nbytes + 2 * GUARD + 256,), CANARY, dtype=torch.uint8, device=device)
            self._pad = (-self.tensor.data_ptr()) % 256 + GUARD
            self.shape = (shape.B, shape.H, shape.d)
            self.io = torch.bfloat16 if shape.dtype == L.SAGE_BF16 else torch.float16

        def check_guards(self):
            B, H, d = self.shape
            rows = B * H * 128 * d
            spans, off = [], 0
            for size in (4, 2, 2):
                spans.append((off, rows * size))
                off = (off + rows * size + 255) // 256 * 256
            # everything after the INT8 rows is the probe's own partial results: one span to the end
            spans.append((off, self.nbytes - off))
            _check_canary(self.tensor, _guard_regions(spans, self._pad, self.nbytes, self.tensor.numel()),
                          "probe scratch")

    return GuardedProbeScratch()


def run_sage(q, k, v, dtype, causal, qk_bits=8, gran="thread", smooth=(True, True, True), p_range=448.0,
             v_range=448.0, layout="bhnd", download=BUFFERS, pv="fp8", qk_format="int"):
    """Quantize and run attention through the C ABI on guarded buffers; checks
    the guards and returns the buffers named in `download` and the output."""
    import torch
    from quantized_attention_sage_amd import api
    qt, kt, vt = (to_device(x, dtype, layout) for x in (q, k, v))
    params = api.make_params(qk_bits=qk_bits, gran=gran, smooth_q=smooth[0], smooth_k=smooth[1], smooth_v=smooth[2],
                             p_range=p_range, v_range=v_range, pv=pv, qk_format=qk_format)
    shape = api.make_shape(qt, kt, vt)
    ws = guarded_workspace(shape, params, qt.device)
    api.quant_qk(qt, kt, vt, params, ws, shape)
    api.quant_v(vt, params, ws, shape)
    g = GuardedOut(qt)
    api.attn_fwd(ws, shape, params, causal, g.out)
    torch.cuda.synchronize()
    ws.check_guards()
    g.check()
    res = {name: ws.view(name).cpu().numpy() for name in download}
    res["out"] = g.out.float().cpu().numpy()
    return res


def unpermute_v(vc: np.ndarray) -> np.ndarray:
    """[B,H,d,n_pad] permuted E4M3 codes -> [B,H,n_pad,d] natural order.

    Within each 64-key group, byte 32h + t holds key 32(t/16) + 8((t%16)/4) + 4h + t%4
    (the layout include/sage.h documents)."""
    n_pad = vc.shape[-1]
    pos = np.empty(64, np.int64)
    for hh in range(2):
        for t in range(32):
            pos[32 * (t // 16) + 8 * ((t % 16) // 4) + 4 * hh + t % 4] = 32 * hh + t
    keys = np.arange(n_pad)
    idx = (keys // 64) * 64 + pos[keys % 64]
    return np.ascontiguousarray(np.swapaxes(vc[..., idx], -1, -2))


def unpermute_v16(vc: np.ndarray) -> np.ndarray:
    """[B,H,d,n_pad] 16-bit V of the 16-bit P~V layout -> [B,H,n_pad,d] uint16, natural order.

    Within each 32-key group, element 16m + 8h + 4a + r holds key 16m + 8a + 4h + r
    (include/sage.h, SAGE_PV_F16): the key offset with bits 2 and 3 swapped."""
    n_pad = vc.shape[-1]
    keys = np.arange(n_pad)
    idx = (keys & ~12) | ((keys & 4) << 1) | ((keys & 8) >> 1)
    return np.ascontiguousarray(np.swapaxes(vc.view(np.uint16)[..., idx], -1, -2))


def half_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of exactly representable float32 values in fp16 / bf16."""
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def assert_quant_bit_exact(gpu: dict, qk: dict, vq: dict):
    np.testing.assert_array_equal(gpu["q_codes"], qk["q_codes"], err_msg="q codes")
    np.testing.assert_array_equal(gpu["k_codes"], qk["k_codes"], err_msg="k codes")
    np.testing.assert_array_equal(bits(gpu["q_scale"]), bits(qk["q_scale"]), err_msg="q scales")
    np.testing.assert_array_equal(bits(gpu["k_scale"]), bits(qk["k_scale"]), err_msg="k scales")
    np.testing.assert_array_equal(bits(gpu["q_mean"]), bits(qk["q_mean"]), err_msg="q means")
    np.testing.assert_array_equal(bits(gpu["k_mean"]), bits(qk["k_mean"]), err_msg="k means")
    np.testing.assert_array_equal(unpermute_v(gpu["v_codes"]), vq["v_codes"], err_msg="v codes")
    np.testing.assert_array_equal(bits(gpu["v_scale"]), bits(vq["v_scale"]), err_msg="v scales")
    np.testing.assert_array_equal(bits(gpu["v_mean"]), bits(vq["v_mean"]), err_msg="v means")


def exp2_scale(d: int) -> float:
    """sm_scale * log2(e) as the library forms it in fp32 (default sm_scale)."""
    return float(np.float32(np.float32(1.0) / np.sqrt(np.float32(d))) * np.float32(1.4426950408889634))


def bias_tolerance_ok(gpu_bias, ref_bias, q_mean, k_smoothed):
    """The library stores dS * sm_scale * log2(e).  dS runs on bf16 matrix cores
    with a 3-product hi/lo split (about 2^-16 relative per product):
    |err| <= (2^-14 * sum_c |mu_c| |K'_jc| + 2^-23 |dS|) * scale."""
    c = exp2_scale(q_mean.shape[-1])
    mag = np.einsum("bhqc,bhjc->bhqj", np.abs(q_mean).astype(np.float64), np.abs(k_smoothed).astype(np.float64))
    ref = ref_bias.astype(np.float64) * c
    err = np.abs(gpu_bias.astype(np.float64) - ref)
    bound = (2.0 ** -14 * mag + 2.0 ** -23 * np.abs(ref_bias)) * c + 1e-30
    return np.all(err <= bound), float((err / bound).max())


def output_tolerance(v: np.ndarray, emul: np.ndarray, dtype: str) -> np.ndarray:
    """2e-3 * max|V| (the bar against the emulation) plus half an output ulp
    for the final rounding of O to fp16/bf16."""
    mant = 8 if dtype == "bf16" else 11
    a = np.abs(emul)
    ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - (mant - 1))
    return 2e-3 * np.abs(v).max() + 0.5 * ulp


def check_output(gpu_out, emul, v, dtype):
    tol = output_tolerance(v, emul, dtype)
    keep = ~np.isnan(emul)
    err = np.abs(gpu_out - emul)
    bad = keep & (err > tol)
    return int(bad.sum()), float(np.nanmax(np.where(keep, err, np.nan))), float(2e-3 * np.abs(v).max())
