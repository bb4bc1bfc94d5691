"""The C-ABI library loads, exports every symbol include/sage.h declares, and its
host-side logic (layout, binding, validation) behaves as documented.  Nothing
here launches a kernel, so it runs without a GPU."""
import ctypes
import os
import re

import pytest

from quantized_attention_sage_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"SAGE_API\s+[\w\s\*]+?\b(sage_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = set(declared_symbols())
    assert {"sage_quant_qk", "sage_quant_v", "sage_attn_fwd", "sage_attn"} <= names
    assert names == set(L.EXPORTS), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {L.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (sage_\w+)", out))
    assert exported == set(declared_symbols())


def test_abi_version_matches_header():
    v = int(re.search(r"#define SAGE_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.lib().sage_abi_version() == v


def _shape(B=1, H=2, N=1000, d=128, dtype=L.SAGE_BF16, stride=None):
    st = stride or (H * N * d, N * d, d)
    return L.Shape(B, H, N, d, dtype, 0, L.c_i64_3(*st), L.c_i64_3(*st), L.c_i64_3(*st))


def _params(**kw):
    p = L.Params()
    L.lib().sage_params_default(ctypes.byref(p))
    for k_, v_ in kw.items():
        setattr(p, k_, v_)
    return p


def test_defaults():
    p = _params()
    assert (p.qk_bits, p.gran, p.smooth_q, p.smooth_k, p.smooth_v) == (8, 0, 1, 1, 1)
    assert (p.p_range, p.v_range, p.sm_scale) == (448.0, 448.0, 0.0)
    assert (p.pv_mode, p.qk_format) == (0, 0)


@pytest.mark.parametrize("gran,gq,gk", [(0, 1024, 64), (1, 32, 16), (2, 8, 16)])
def test_layout_sizes(gran, gq, gk):
    B, H, N, d = 2, 3, 1000, 128
    n_pad, nblk = 1024, 8
    lay = L.Layout()
    assert L.lib().sage_workspace_layout(ctypes.byref(_shape(B, H, N, d)), ctypes.byref(_params(gran=gran)),
                                         ctypes.byref(lay)) == L.SAGE_OK
    assert (lay.n_pad, lay.n_qblocks, lay.q_groups, lay.k_groups) == (n_pad, nblk, gq, gk)
    BH = B * H
    expect = {"q_codes": BH * n_pad * d, "k_codes": BH * n_pad * d, "q_scale": BH * gq * 4, "k_scale": BH * gk * 4,
              "q_mean": BH * nblk * d * 4, "k_mean": BH * d * 4, "bias": BH * nblk * n_pad * 4,
              "k_partial": BH * nblk * d * 4, "v_codes": BH * d * n_pad, "v_scale": BH * d * 4,
              "v_mean": BH * d * 4, "v_partial": BH * nblk * 3 * d * 4}
    spans = sorted((getattr(lay, n).offset, getattr(lay, n).bytes, n) for n in L.SPANS)
    for (off, size, name) in spans:
        assert size == expect[name], name
        assert off % 256 == 0
    for (a, b) in zip(spans, spans[1:]):
        assert a[0] + a[1] <= b[0]
    assert spans[-1][0] + spans[-1][1] <= lay.total_bytes


def test_bwd_layout_sizes():
    """Every span of the backward workspace has the size include/sage.h states,
    is 256-byte aligned and overlaps no other."""
    B, H, N, d = 2, 3, 1000, 128
    n_pad, nblk, BH = 1024, 8, 6
    lay = L.BwdLayout()
    assert L.lib().sage_bwd_workspace_layout(ctypes.byref(_shape(B, H, N, d)), ctypes.byref(_params()),
                                             ctypes.byref(lay)) == L.SAGE_OK
    assert lay.n_pad == n_pad
    row = BH * n_pad * 4
    expect = {"do_codes": BH * n_pad * d, "do_scale": row, "do_mean": BH * nblk * d * 4,
              "v_codes": BH * n_pad * d, "v_scale": BH * (n_pad // 16) * 4, "v_mean": BH * d * 4,
              "v_partial": BH * nblk * d * 4, "fp8_partial": BH * nblk * 3 * d * 4,
              "dsum": row, "lse_do": row, "dsum_do": row}
    for n in ("do8", "q8", "k8"):
        expect.update({f"{n}_codes": BH * d * n_pad, f"{n}_scale": BH * d * 4, f"{n}_mean": BH * d * 4})
    assert set(expect) == set(L.BWD_SPANS)
    spans = sorted((getattr(lay, n).offset, getattr(lay, n).bytes, n) for n in L.BWD_SPANS)
    for (off, size, name) in spans:
        assert size == expect[name], name
        assert off % 256 == 0
    for (a, b) in zip(spans, spans[1:]):
        assert a[0] + a[1] <= b[0]
    assert spans[-1][0] + spans[-1][1] <= lay.total_bytes


@pytest.mark.parametrize("mode", ["mxfp4", "pv16", "int_e4m3", "int_e2m3"])
def test_layout_sizes_other_formats(mode):
    """MXFP4 codes are 4 bits (d/2 bytes per token) with one scale byte per 32
    channels; the 16-bit P~V keeps V itself (2 bytes per element); E4M3-held
    INT4-range codes take the INT layout byte for byte."""
    B, H, N, d = 2, 3, 1000, 128
    n_pad, BH = 1024, 6
    kw = {"mxfp4": dict(qk_format=1), "pv16": dict(pv_mode=1), "int_e4m3": dict(qk_format=2, qk_bits=4),
          "int_e2m3": dict(qk_format=3, qk_bits=4)}[mode]
    lay = L.Layout()
    assert L.lib().sage_workspace_layout(ctypes.byref(_shape(B, H, N, d)), ctypes.byref(_params(**kw)),
                                         ctypes.byref(lay)) == L.SAGE_OK
    if mode == "mxfp4":
        assert lay.q_codes.bytes == lay.k_codes.bytes == BH * n_pad * d // 2
        assert lay.q_scale.bytes == lay.k_scale.bytes == BH * n_pad * d // 32
        assert lay.v_codes.bytes == BH * d * n_pad
    elif mode in ("int_e4m3", "int_e2m3"):
        ref = L.Layout()
        L.lib().sage_workspace_layout(ctypes.byref(_shape(B, H, N, d)), ctypes.byref(_params(qk_bits=4)),
                                      ctypes.byref(ref))
        for n in L.SPANS:
            assert (getattr(lay, n).offset, getattr(lay, n).bytes) == (getattr(ref, n).offset, getattr(ref, n).bytes)
    else:
        assert lay.q_codes.bytes == BH * n_pad * d and lay.v_codes.bytes == 2 * BH * d * n_pad


def test_bind_workspace_checks():
    lib = L.lib()
    lay = L.Layout()
    lib.sage_workspace_layout(ctypes.byref(_shape()), ctypes.byref(_params()), ctypes.byref(lay))
    qk, vb = L.QKBuffers(), L.VBuffers()
    base = 1 << 40   # never dereferenced
    assert lib.sage_bind_workspace(ctypes.byref(lay), ctypes.c_void_p(base + 16), lay.total_bytes,
                                   ctypes.byref(qk), ctypes.byref(vb)) == L.SAGE_EINVAL
    assert lib.sage_bind_workspace(ctypes.byref(lay), ctypes.c_void_p(base), lay.total_bytes - 1,
                                   ctypes.byref(qk), ctypes.byref(vb)) == L.SAGE_EINVAL
    assert b"too small" in lib.sage_last_error()
    assert lib.sage_bind_workspace(ctypes.byref(lay), ctypes.c_void_p(base), lay.total_bytes,
                                   ctypes.byref(qk), ctypes.byref(vb)) == L.SAGE_OK
    assert qk.bias == base + lay.bias.offset and vb.v_codes == base + lay.v_codes.offset


BAD_SHAPES = [
    dict(d=96), dict(N=0), dict(N=(1 << 20) + 1), dict(B=0), dict(dtype=7),
    dict(stride=(1000 * 128 * 2, 1000 * 128, 100)),      # N stride not a multiple of 8
    dict(stride=(1000 * (1 << 22) * 2, 1000 * (1 << 22), 1 << 22)),   # N stride at the 2^22-element limit
]


@pytest.mark.parametrize("bad", BAD_SHAPES)
def test_bad_shapes_are_rejected(bad):
    lay = L.Layout()
    st = L.lib().sage_workspace_layout(ctypes.byref(_shape(**bad)), ctypes.byref(_params()), ctypes.byref(lay))
    assert st in (L.SAGE_EINVAL, L.SAGE_EUNSUPPORTED)
    assert L.lib().sage_last_error() != b""


BAD_PARAMS = [dict(qk_bits=6), dict(gran=3), dict(smooth_q=2), dict(p_range=0.0), dict(p_range=449.0),
              dict(v_range=-1.0), dict(sm_scale=-0.5), dict(sm_scale=float("inf")), dict(pv_mode=2),
              dict(qk_format=5), dict(qk_format=1, pv_mode=1),
              dict(qk_format=2), dict(qk_format=2, qk_bits=4, pv_mode=1),   # E4M3-held codes: INT4-range, FP8 P~V
              dict(qk_format=3), dict(qk_format=3, qk_bits=4, pv_mode=1), dict(qk_format=4)]


@pytest.mark.parametrize("bad", BAD_PARAMS)
def test_bad_params_are_rejected(bad):
    lay = L.Layout()
    st = L.lib().sage_workspace_layout(ctypes.byref(_shape()), ctypes.byref(_params(**bad)), ctypes.byref(lay))
    assert st in (L.SAGE_EINVAL, L.SAGE_EUNSUPPORTED)


def test_entry_points_validate_before_launching():
    lib = L.lib()
    sh, p = _shape(), _params()
    fake = ctypes.c_void_p(1 << 40)
    qk = L.QKBuffers(*([1 << 40] * 8))
    vb = L.VBuffers(*([1 << 40] * 4))
    strides = (ctypes.c_int64 * 3)(256000, 128000, 128)
    assert lib.sage_quant_qk(None, fake, ctypes.byref(sh), ctypes.byref(p), ctypes.byref(qk), None) == L.SAGE_EINVAL
    assert lib.sage_quant_qk(fake, ctypes.c_void_p((1 << 40) + 2), ctypes.byref(sh), ctypes.byref(p),
                             ctypes.byref(qk), None) == L.SAGE_EINVAL     # misaligned
    qk_null = L.QKBuffers(*([1 << 40] * 7 + [0]))
    assert lib.sage_quant_qk(fake, fake, ctypes.byref(sh), ctypes.byref(p), ctypes.byref(qk_null),
                             None) == L.SAGE_EINVAL
    assert lib.sage_quant_v(fake, ctypes.byref(sh), ctypes.byref(_params(v_range=500.0)), ctypes.byref(vb),
                            None) == L.SAGE_EINVAL
    assert lib.sage_attn_fwd(ctypes.byref(qk), ctypes.byref(vb), ctypes.byref(sh), ctypes.byref(p), 2, fake,
                             strides, None) == L.SAGE_EINVAL                # causal must be 0/1
    bad_strides = (ctypes.c_int64 * 3)(256000, 128000, 130)
    assert lib.sage_attn_fwd(ctypes.byref(qk), ctypes.byref(vb), ctypes.byref(sh), ctypes.byref(p), 0, fake,
                             bad_strides, None) == L.SAGE_EINVAL
    assert lib.sage_attn(fake, fake, fake, ctypes.byref(sh), ctypes.byref(p), 0, fake, strides, fake, 10,
                         None) == L.SAGE_EINVAL                            # workspace too small
    assert lib.sage_status_str(L.SAGE_EUNSUPPORTED) == b"unsupported"


def test_static_entry_validates_before_launching():
    """sage_attn_static rejects on the host, before touching any device: a
    problem whose workspace exceeds the static array, and bad arguments."""
    lib = L.lib()
    p = _params()
    fake = ctypes.c_void_p(1 << 40)
    N, H = 8192, 16                                             # about 83 MiB of workspace
    st = (ctypes.c_int64 * 3)(H * N * 128, N * 128, 128)
    big = L.Shape(1, H, N, 128, L.SAGE_BF16, 0, L.c_i64_3(*st), L.c_i64_3(*st), L.c_i64_3(*st))
    assert lib.sage_attn_static(fake, fake, fake, ctypes.byref(big), ctypes.byref(p), 0, fake, st,
                                None) == L.SAGE_EUNSUPPORTED
    assert b"static" in lib.sage_last_error()
    sh = _shape()
    strides = (ctypes.c_int64 * 3)(256000, 128000, 128)
    assert lib.sage_attn_static(None, fake, fake, ctypes.byref(sh), ctypes.byref(p), 0, fake, strides,
                                None) == L.SAGE_EINVAL
    assert lib.sage_attn_static(fake, fake, fake, ctypes.byref(sh), ctypes.byref(p), 2, fake, strides,
                                None) == L.SAGE_EINVAL                # causal must be 0/1
    assert L.STATIC_WORKSPACE_BYTES == int(re.search(r"#define SAGE_STATIC_WORKSPACE_BYTES \((\d+)u << (\d+)\)",
                                                     open(HEADER).read()).group(1)) << 20


def test_probe_scratch_bytes():
    """Exact rows fp32, two outputs of the I/O type, per-split partial rows
    (at most 64 splits of whole 8-key sub-tiles, 1024 keys up to 64K keys)
    and the fp64 sums, each span 256-byte aligned."""
    def al(x):
        return (x + 255) // 256 * 256
    for (B, H, N, d) in [(2, 3, 1000, 128), (1, 32, 16384, 128), (1, 2, 1 << 20, 64)]:
        n = ctypes.c_size_t()
        assert L.lib().sage_probe_scratch_bytes(ctypes.byref(_shape(B, H, N, d)), ctypes.byref(n)) == L.SAGE_OK
        BH, n_pad = B * H, (N + 127) // 128 * 128
        chunk = 1024 if n_pad <= 64 * 1024 else ((n_pad + 63) // 64 + 7) // 8 * 8
        S = -(-n_pad // chunk)
        assert S <= 64
        want = al(BH * 128 * d * 4) + 2 * al(BH * 128 * d * 2) + al(S * BH * 128 * (d + 2) * 4) + al(BH * 64) + al(64)
        assert n.value == want


BAD_PROBES = [dict(q_block=-1), dict(q_block=8), dict(qk_format=1), dict(pv_mode=1), dict(cos_min=float("nan")),
              dict(scratch_bytes=-1), dict(result=False), dict(causal=2)]


@pytest.mark.parametrize("bad", BAD_PROBES)
def test_probe_validates_before_launching(bad):
    """Every bad argument is refused with no device access (the pointers are
    never dereferenced)."""
    lib = L.lib()
    shape = _shape()       # N = 1000: 8 query blocks
    lay = L.Layout()
    kw = {k: v for k, v in bad.items() if k in ("qk_format", "pv_mode")}
    params = _params(qk_bits=4, **kw)
    lay_params = _params(qk_bits=4)
    assert lib.sage_workspace_layout(ctypes.byref(shape), ctypes.byref(lay_params), ctypes.byref(lay)) == L.SAGE_OK
    qk, vb = L.QKBuffers(), L.VBuffers()
    base = 1 << 40
    assert lib.sage_bind_workspace(ctypes.byref(lay), ctypes.c_void_p(base), lay.total_bytes, ctypes.byref(qk),
                                   ctypes.byref(vb)) == L.SAGE_OK
    n = ctypes.c_size_t()
    lib.sage_probe_scratch_bytes(ctypes.byref(shape), ctypes.byref(n))
    scratch_bytes = n.value + (bad["scratch_bytes"] if "scratch_bytes" in bad else 0)
    res = L.ProbeResult()
    st = lib.sage_probe_qk_bits(ctypes.c_void_p(base), ctypes.c_void_p(base), ctypes.c_void_p(base),
                                ctypes.byref(shape), ctypes.byref(params), bad.get("causal", 0), bad.get("q_block", 0),
                                bad.get("cos_min", 0.999), ctypes.byref(qk), ctypes.byref(vb),
                                ctypes.c_void_p(base + (1 << 36)), scratch_bytes,
                                ctypes.byref(res) if bad.get("result", True) else None, None)
    assert st in (L.SAGE_EINVAL, L.SAGE_EUNSUPPORTED)
    assert lib.sage_last_error() != b""

