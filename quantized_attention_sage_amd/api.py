"""Torch-facing wrappers of the C ABI (memory and streams only).

PyTorch provides device memory and the current HIP stream; the wrappers pass
raw pointers, sizes and the stream to libsage.so and return views of the
buffers it wrote.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L

_DTYPES = {torch.float16: L.SAGE_F16, torch.bfloat16: L.SAGE_BF16}


def make_params(qk_bits: int = 8, gran: str = "thread", smooth_q: bool = True, smooth_k: bool = True,
                smooth_v: bool = True, p_range: float = 448.0, v_range: float = 448.0,
                sm_scale: float = 0.0, pv: str = "fp8", qk_format: str = "int") -> L.Params:
    if gran not in L.GRAN:
        raise ValueError(f"granularity must be one of {sorted(L.GRAN)}")
    if pv not in L.PV_MODE:
        raise ValueError(f"pv must be one of {sorted(L.PV_MODE)}")
    if qk_format not in L.QK_FORMAT:
        raise ValueError(f"qk_format must be one of {sorted(L.QK_FORMAT)}")
    return L.Params(int(qk_bits), L.GRAN[gran], int(bool(smooth_q)), int(bool(smooth_k)), int(bool(smooth_v)),
                    float(p_range), float(v_range), float(sm_scale), L.PV_MODE[pv], L.QK_FORMAT[qk_format])


def _check_tensor(x: torch.Tensor, name: str):
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d]")
    if x.dtype not in _DTYPES:
        raise TypeError(f"{name} must be float16 or bfloat16")
    if x.stride(3) != 1:
        raise ValueError(f"{name} must be contiguous in d")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")


def make_shape(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> L.Shape:
    for x, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(x, n)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    B, H, N, d = q.shape
    return L.Shape(B, H, N, d, _DTYPES[q.dtype], 0, L.c_i64_3(*q.stride()[:3]), L.c_i64_3(*k.stride()[:3]),
                   L.c_i64_3(*v.stride()[:3]))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Workspace:
    """One device allocation holding every intermediate buffer, with typed views."""

    def __init__(self, shape: L.Shape, params: L.Params, device):
        lay = L.Layout()
        L.check(L.lib().sage_workspace_layout(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(lay)))
        self.layout = lay
        self.shape = (shape.B, shape.H, shape.N, shape.d)
        self.pv_f16 = params.pv_mode == L.PV_MODE["f16"]
        self.qk_mx = params.qk_format == L.QK_FORMAT["mxfp4"]
        self.qk_held = params.qk_format in (L.QK_FORMAT["int_e4m3"], L.QK_FORMAT["int_e2m3"])
        self.tensor = torch.empty(lay.total_bytes + 256, dtype=torch.uint8, device=device)
        base = self.tensor.data_ptr()
        self._pad = (-base) % 256
        self.qk = L.QKBuffers()
        self.vb = L.VBuffers()
        L.check(L.lib().sage_bind_workspace(ctypes.byref(lay), ctypes.c_void_p(base + self._pad),
                                            ctypes.c_size_t(lay.total_bytes), ctypes.byref(self.qk),
                                            ctypes.byref(self.vb)))

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr() + self._pad

    @property
    def nbytes(self) -> int:
        return self.layout.total_bytes

    def view(self, name: str) -> torch.Tensor:
        """Typed view of one buffer, shaped as include/sage.h documents it."""
        B, H, N, d = self.shape
        lay = self.layout
        n_pad, nblk = lay.n_pad, lay.n_qblocks
        sp = getattr(lay, name)
        code_t = torch.uint8 if self.qk_held else torch.int8     # E4M3 / packed E2M3 bytes, or int8 codes
        raw = self.tensor[self._pad + sp.offset: self._pad + sp.offset + sp.bytes]
        shapes = {
            "q_codes": (torch.uint8, (B, H, n_pad, d // 2)) if self.qk_mx else (code_t, (B, H, n_pad, d)),
            "k_codes": (torch.uint8, (B, H, n_pad, d // 2)) if self.qk_mx else (code_t, (B, H, n_pad, d)),
            "q_scale": (torch.uint8, (B, H, n_pad, d // 32)) if self.qk_mx else (torch.float32, (B, H, lay.q_groups)),
            "k_scale": (torch.uint8, (B, H, n_pad, d // 32)) if self.qk_mx else (torch.float32, (B, H, lay.k_groups)),
            "q_mean": (torch.float32, (B, H, nblk, d)),
            "k_mean": (torch.float32, (B, H, d)),
            "bias": (torch.float32, (B, H, nblk, n_pad)),
            "k_partial": (torch.float32, (B, H, nblk, d)),
            "v_codes": (torch.int16 if self.pv_f16 else torch.uint8, (B, H, d, n_pad)),
            "v_scale": (torch.float32, (B, H, d)),
            "v_mean": (torch.float32, (B, H, d)),
            "v_partial": (torch.float32, (B, H, nblk, 3, d)),
        }
        dt, shp = shapes[name]
        return raw.view(dt).view(shp)


def quant_qk(q, k, v_for_shape, params: L.Params, ws: Workspace, shape: L.Shape = None):
    shape = shape or make_shape(q, k, v_for_shape)
    L.check(L.lib().sage_quant_qk(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.byref(shape),
                                  ctypes.byref(params), ctypes.byref(ws.qk), ctypes.c_void_p(_stream(q.device))))


def quant_v(v, params: L.Params, ws: Workspace, shape: L.Shape):
    L.check(L.lib().sage_quant_v(ctypes.c_void_p(v.data_ptr()), ctypes.byref(shape), ctypes.byref(params),
                                 ctypes.byref(ws.vb), ctypes.c_void_p(_stream(v.device))))


def _out_strides(o: torch.Tensor):
    return (ctypes.c_int64 * 3)(*o.stride()[:3])


def attn_fwd(ws: Workspace, shape: L.Shape, params: L.Params, causal: bool, out: torch.Tensor):
    _check_tensor(out, "out")
    L.check(L.lib().sage_attn_fwd(ctypes.byref(ws.qk), ctypes.byref(ws.vb), ctypes.byref(shape), ctypes.byref(params),
                                  int(bool(causal)), ctypes.c_void_p(out.data_ptr()), _out_strides(out),
                                  ctypes.c_void_p(_stream(out.device))))


def attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, out: torch.Tensor = None,
         workspace: Workspace = None, **kw) -> torch.Tensor:
    """Plug-and-play quantized attention: O = softmax(sm_scale Q K^T [+ causal mask]) V.

    Keyword arguments are those of ``make_params``.  Returns ``out`` (allocated
    like ``q`` when not given).
    """
    params = make_params(**kw)
    shape = make_shape(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out")
    ws = workspace or Workspace(shape, params, q.device)
    L.check(L.lib().sage_attn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                              ctypes.c_void_p(v.data_ptr()), ctypes.byref(shape), ctypes.byref(params),
                              int(bool(causal)), ctypes.c_void_p(out.data_ptr()), _out_strides(out),
                              ctypes.c_void_p(ws.ptr), ctypes.c_size_t(ws.nbytes), ctypes.c_void_p(_stream(q.device))))
    return out


def attn_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, out: torch.Tensor = None,
                **kw) -> torch.Tensor:
    """``attn`` with every intermediate in the library-held static workspace
    (sage_attn_static): no device allocation by the library.  ``out`` is
    allocated like ``q`` only when not given."""
    params = make_params(**kw)
    shape = make_shape(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out")
    L.check(L.lib().sage_attn_static(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                     ctypes.c_void_p(v.data_ptr()), ctypes.byref(shape), ctypes.byref(params),
                                     int(bool(causal)), ctypes.c_void_p(out.data_ptr()), _out_strides(out),
                                     ctypes.c_void_p(_stream(q.device))))
    return out


def attn_fwd_lse(ws: Workspace, shape: L.Shape, params: L.Params, causal: bool, out: torch.Tensor,
                 lse: torch.Tensor):
    """attn_fwd that also writes lse (float32 [B, H, N_pad]): log2 sum_j 2^(s_ij)."""
    _check_tensor(out, "out")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != shape.B * shape.H * ws.layout.n_pad:
        raise ValueError("lse must be a contiguous float32 [B, H, N_pad] tensor")
    L.check(L.lib().sage_attn_fwd_lse(ctypes.byref(ws.qk), ctypes.byref(ws.vb), ctypes.byref(shape),
                                      ctypes.byref(params), int(bool(causal)), ctypes.c_void_p(out.data_ptr()),
                                      _out_strides(out), ctypes.c_void_p(lse.data_ptr()),
                                      ctypes.c_void_p(_stream(out.device))))


class BwdWorkspace:
    """The backward's intermediate buffers in one device allocation, with views."""

    def __init__(self, shape: L.Shape, params: L.Params, device):
        lay = L.BwdLayout()
        L.check(L.lib().sage_bwd_workspace_layout(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(lay)))
        self.layout = lay
        self.shape = (shape.B, shape.H, shape.N, shape.d)
        self.tensor = torch.empty(lay.total_bytes + 256, dtype=torch.uint8, device=device)
        self._pad = (-self.tensor.data_ptr()) % 256

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr() + self._pad

    @property
    def nbytes(self) -> int:
        return self.layout.total_bytes

    def view(self, name: str) -> torch.Tensor:
        B, H, N, d = self.shape
        n_pad = self.layout.n_pad
        sp = getattr(self.layout, name)
        raw = self.tensor[self._pad + sp.offset: self._pad + sp.offset + sp.bytes]
        shapes = {
            "do_codes": (torch.int8, (B, H, n_pad, d)), "do_scale": (torch.float32, (B, H, n_pad)),
            "v_codes": (torch.int8, (B, H, n_pad, d)), "v_scale": (torch.float32, (B, H, n_pad // 16)),
            "do8_codes": (torch.uint8, (B, H, d, n_pad)), "do8_scale": (torch.float32, (B, H, d)),
            "q8_codes": (torch.uint8, (B, H, d, n_pad)), "q8_scale": (torch.float32, (B, H, d)),
            "k8_codes": (torch.uint8, (B, H, d, n_pad)), "k8_scale": (torch.float32, (B, H, d)),
            "k8_mean": (torch.float32, (B, H, d)), "dsum": (torch.float32, (B, H, n_pad)),
            "lse_do": (torch.float32, (B, H, n_pad)), "dsum_do": (torch.float32, (B, H, n_pad)),
        }
        dt, shp = shapes[name]
        return raw.view(dt).view(shp)


def attn_bwd(q, k, v, o, dout, lse: torch.Tensor, ws: Workspace, shape: L.Shape, params: L.Params, causal: bool,
             bws: BwdWorkspace, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor):
    """The 8-bit backward: writes float32 dq, dk, dv ([B, H, N, d], contiguous)."""
    for t_, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t_.dtype != torch.float32 or not t_.is_contiguous() or tuple(t_.shape) != tuple(q.shape):
            raise ValueError(f"{n} must be a contiguous float32 tensor shaped like q")
    if o.stride() != dout.stride():
        raise ValueError("o and dout must share strides")
    L.check(L.lib().sage_attn_bwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                  ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                                  ctypes.c_void_p(dout.data_ptr()), _out_strides(o), ctypes.c_void_p(lse.data_ptr()),
                                  ctypes.byref(ws.qk), ctypes.byref(shape), ctypes.byref(params), int(bool(causal)),
                                  ctypes.c_void_p(dq.data_ptr()), ctypes.c_void_p(dk.data_ptr()),
                                  ctypes.c_void_p(dv.data_ptr()), ctypes.c_void_p(bws.ptr),
                                  ctypes.c_size_t(bws.nbytes), ctypes.c_void_p(_stream(q.device))))


class ProbeScratch:
    """Device scratch of the adaptive INT4/INT8 probe, with views of the probed rows."""

    def __init__(self, shape: L.Shape, device):
        n = ctypes.c_size_t()
        L.check(L.lib().sage_probe_scratch_bytes(ctypes.byref(shape), ctypes.byref(n)))
        self.nbytes = n.value
        self.tensor = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        self._pad = (-self.tensor.data_ptr()) % 256
        self.shape = (shape.B, shape.H, shape.d)
        self.io = torch.bfloat16 if shape.dtype == L.SAGE_BF16 else torch.float16

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr() + self._pad

    def rows(self):
        """(exact fp32, INT4-range, INT8) rows [B, H, 128, d] as the probe left them."""
        B, H, d = self.shape
        n = B * H * 128 * d
        off, out = 0, []
        for dt, size in ((torch.float32, 4), (self.io, 2), (self.io, 2)):
            raw = self.tensor[self._pad + off: self._pad + off + n * size]
            out.append(raw.view(dt).view(B, H, 128, d))
            off = (off + n * size + 255) // 256 * 256
        return tuple(out)


def probe_qk_bits(q, k, v, params: L.Params, ws: Workspace, shape: L.Shape, causal: bool, q_block: int,
                  cos_min: float, scratch: ProbeScratch = None) -> dict:
    """Adaptive INT4/INT8 choice on query block ``q_block`` of every head.

    Leaves the quantisation of the chosen precision in ``ws``; returns the
    metrics of both precisions and ``qk_bits``."""
    scratch = scratch or ProbeScratch(shape, q.device)
    res = L.ProbeResult()
    L.check(L.lib().sage_probe_qk_bits(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                       ctypes.c_void_p(v.data_ptr()), ctypes.byref(shape), ctypes.byref(params),
                                       int(bool(causal)), int(q_block), float(cos_min), ctypes.byref(ws.qk),
                                       ctypes.byref(ws.vb), ctypes.c_void_p(scratch.ptr),
                                       ctypes.c_size_t(scratch.nbytes), ctypes.byref(res),
                                       ctypes.c_void_p(_stream(q.device))))
    return {"cos_int4": res.cos_int4, "cos_int8": res.cos_int8, "rel_l1_int4": res.rel_l1_int4,
            "rel_l1_int8": res.rel_l1_int8, "qk_bits": res.qk_bits}

