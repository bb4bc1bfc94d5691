"""SageAttention2-style quantized attention forward pass for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``include/sage.h`` (``libsage.so`` in this folder).  This package holds the
ctypes binding (``_lib``), torch-facing wrappers that pass device pointers and
the current stream (``api``), the build step (``build``) and the seeded
synthetic workloads (``workloads``).
"""
from ._lib import SageError, lib, LIB_PATH  # noqa: F401


def __getattr__(name):
    # torch-facing wrappers are imported lazily so that `workloads` and `build`
    # stay usable without touching the GPU runtime.
    if name in ("attn", "attn_fwd", "quant_qk", "quant_v", "make_params", "make_shape", "Workspace"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
