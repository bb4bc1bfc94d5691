"""ctypes mirror of include/sage.h and the loader of libsage.so.

Only argument marshalling lives here; every step of the computation runs in
the HIP kernels behind the C ABI.  There is no fallback: if the library is
missing or cannot be loaded, import of the binding fails with an error.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# SAGE_LIBRARY names another build of the same ABI (the host-sanitizer test
# loads one); by default the in-tree libsage.so.
LIB_PATH = os.environ.get("SAGE_LIBRARY") or os.path.join(PKG, "libsage.so")

SAGE_OK, SAGE_EINVAL, SAGE_EUNSUPPORTED, SAGE_EHIP = 0, 1, 2, 3
SAGE_F16, SAGE_BF16 = 0, 1
GRAN = {"thread": 0, "warp": 1, "block": 2}
PV_MODE = {"fp8": 0, "f16": 1}
QK_FORMAT = {"int": 0, "mxfp4": 1, "int_e4m3": 2, "int_e2m3": 3}
ABI_VERSION = 7
STATIC_WORKSPACE_BYTES = 64 << 20   # SAGE_STATIC_WORKSPACE_BYTES

c_i64_3 = ctypes.c_int64 * 3


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64), ("d", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("q_stride", c_i64_3), ("k_stride", c_i64_3), ("v_stride", c_i64_3)]


class Params(ctypes.Structure):
    _fields_ = [("qk_bits", ctypes.c_int32), ("gran", ctypes.c_int32), ("smooth_q", ctypes.c_int32),
                ("smooth_k", ctypes.c_int32), ("smooth_v", ctypes.c_int32), ("p_range", ctypes.c_float),
                ("v_range", ctypes.c_float), ("sm_scale", ctypes.c_float), ("pv_mode", ctypes.c_int32),
                ("qk_format", ctypes.c_int32)]


class QKBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q_codes", "q_scale", "q_mean", "k_codes", "k_scale", "k_mean", "bias", "k_partial")]


class VBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("v_codes", "v_scale", "v_mean", "v_partial")]


class Span(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_size_t), ("bytes", ctypes.c_size_t)]


SPANS = ("q_codes", "q_scale", "q_mean", "k_codes", "k_scale", "k_mean", "bias", "k_partial",
         "v_codes", "v_scale", "v_mean", "v_partial")


class Layout(ctypes.Structure):
    _fields_ = ([("n_pad", ctypes.c_int64), ("n_qblocks", ctypes.c_int64), ("q_groups", ctypes.c_int64),
                 ("k_groups", ctypes.c_int64)] + [(n, Span) for n in SPANS] + [("total_bytes", ctypes.c_size_t)])


BWD_SPANS = ("do_codes", "do_scale", "do_mean", "v_codes", "v_scale", "v_mean", "v_partial",
             "do8_codes", "do8_scale", "do8_mean", "q8_codes", "q8_scale", "q8_mean", "k8_codes", "k8_scale",
             "k8_mean", "fp8_partial", "dsum", "lse_do", "dsum_do")


class BwdLayout(ctypes.Structure):
    _fields_ = [("n_pad", ctypes.c_int64)] + [(n, Span) for n in BWD_SPANS] + [("total_bytes", ctypes.c_size_t)]


class ProbeResult(ctypes.Structure):
    _fields_ = [("cos_int4", ctypes.c_double), ("cos_int8", ctypes.c_double), ("rel_l1_int4", ctypes.c_double),
                ("rel_l1_int8", ctypes.c_double), ("qk_bits", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SageError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sage status {status}: {message}")
        self.status = status


_LIB = None

EXPORTS = {
    "sage_abi_version": (ctypes.c_int, []),
    "sage_params_default": (None, [ctypes.POINTER(Params)]),
    "sage_workspace_layout": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(Params), ctypes.POINTER(Layout)]),
    "sage_bind_workspace": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.POINTER(QKBuffers), ctypes.POINTER(VBuffers)]),
    "sage_quant_qk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.POINTER(Params),
                                     ctypes.POINTER(QKBuffers), ctypes.c_void_p]),
    "sage_quant_v": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.POINTER(Params),
                                    ctypes.POINTER(VBuffers), ctypes.c_void_p]),
    "sage_attn_fwd": (ctypes.c_int, [ctypes.POINTER(QKBuffers), ctypes.POINTER(VBuffers), ctypes.POINTER(Shape),
                                     ctypes.POINTER(Params), ctypes.c_int, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]),
    "sage_attn": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Shape),
                                 ctypes.POINTER(Params), ctypes.c_int, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "sage_attn_static": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Shape),
                                        ctypes.POINTER(Params), ctypes.c_int, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]),
    "sage_attn_fwd_lse": (ctypes.c_int, [ctypes.POINTER(QKBuffers), ctypes.POINTER(VBuffers), ctypes.POINTER(Shape),
                                         ctypes.POINTER(Params), ctypes.c_int, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p, ctypes.c_void_p]),
    "sage_bwd_workspace_layout": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(Params),
                                                 ctypes.POINTER(BwdLayout)]),
    "sage_attn_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p,
                                     ctypes.POINTER(QKBuffers), ctypes.POINTER(Shape), ctypes.POINTER(Params),
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "sage_probe_scratch_bytes": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)]),
    "sage_probe_qk_bits": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Shape),
                                          ctypes.POINTER(Params), ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                          ctypes.POINTER(QKBuffers), ctypes.POINTER(VBuffers), ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.POINTER(ProbeResult), ctypes.c_void_p]),
    "sage_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "sage_last_error": (ctypes.c_char_p, []),
}


def lib():
    """Load libsage.so once (raises if it was not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m quantized_attention_sage_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(status: int):
    if status != SAGE_OK:
        raise SageError(status, lib().sage_last_error().decode())
