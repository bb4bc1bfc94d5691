"""Build libsage.so (HIP kernels for gfx950 + the C ABI) in the package folder.

    python -m quantized_attention_sage_amd.build

Every source is compiled with hipcc for gfx950 only.  The quantisation
kernels are compiled without floating-point contraction (their fp32 results
decide integer and FP8 codes and must be exactly reproducible).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsage.so")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-fvisibility=hidden",
          "-I", INCLUDE, "-I", CSRC,
          # packed fp32 arithmetic stays off: plain v_fma/v_mul/v_add only
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = {
    "quant.hip": ["-ffp-contract=off"],
    "attn.hip": [],
    "attn_pvh.hip": [],
    "attn_fp4.hip": [],
    "probe.hip": [],
    "sage_api.cpp": ["-x", "hip"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="sage_build_") as tmp:
        objs = []
        for src, extra in SOURCES.items():
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
            out = _run(cmd)
            if verbose and out.strip():
                print(out)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libsage.so")
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs)
        os.replace(tmp_lib, LIB) if os.path.dirname(tmp_lib) == os.path.dirname(LIB) else shutil.move(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
