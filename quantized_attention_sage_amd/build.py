"""Build libsage.so (HIP kernels for gfx950 + the C ABI) in the package folder.

    python -m quantized_attention_sage_amd.build

Every source is compiled with hipcc for gfx950 only.  The quantisation
kernels are compiled without floating-point contraction (their fp32 results
decide integer and FP8 codes and must be exactly reproducible).

The attention kernels wait for their own global-to-LDS copies by count
(s_waitcnt vmcnt).  A register spill inside their key loop would add compiler
memory operations to those counts (which only makes the waits stricter, but
costs a full wait for every reload), so the build reads the gfx950 assembly of
each attention source and fails if a scratch access sits inside a loop.
"""
from __future__ import annotations

import os
import re
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
# sources whose kernels must keep scratch accesses out of every loop
LOOP_SPILL_FREE = ("attn.hip", "attn_pvh.hip", "attn_fp4.hip")
SOURCES = {
    "quant.hip": ["-ffp-contract=off"],
    "attn.hip": [],
    "attn_pvh.hip": [],
    "attn_fp4.hip": [],
    "probe.hip": [],
    "static_ws.hip": [],
    "sage_api.cpp": ["-x", "hip"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, cwd=None):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, cwd=cwd)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


def loops_with_scratch(asm: str) -> list:
    """(kernel, first line, last line, scratch ops) of every loop of every kernel
    in a gfx950 assembly listing that contains a scratch access.  A loop is the
    span from a branch target label to a later branch back to it."""
    bad = []
    func, labels = None, {}
    lines = asm.splitlines()
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            func, labels = m.group(1), {}
            continue
        if func is None:
            continue
        if line.startswith(".Lfunc_end"):
            func = None
            continue
        m = re.match(r"^(\.LBB\S+):", line)
        if m:
            labels[m.group(1)] = i
            continue
        m = re.match(r"^\s+s_(?:cbranch_\w+|branch)\s+(\.LBB\S+)", line)
        if m and m.group(1) in labels:
            lo = labels[m.group(1)]
            n = sum(1 for j in range(lo, i) if re.match(r"^\s+scratch_", lines[j]))
            if n:
                bad.append((func, lo + 1, i + 1, n))
    return bad


def _compile(cc: str, tmp: str, src: str, extra: list) -> tuple:
    obj = os.path.join(tmp, src + ".o")
    temps = ["-save-temps"] if src in LOOP_SPILL_FREE else []
    # each source gets its own folder: -save-temps writes its files to the working directory
    wd = os.path.join(tmp, src + ".d")
    os.makedirs(wd)
    out = _run([cc] + COMMON + extra + temps + ["-c", os.path.join(CSRC, src), "-o", obj], cwd=wd)
    if temps:
        stem = os.path.splitext(src)[0]
        with open(os.path.join(wd, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s")) as fh:
            bad = loops_with_scratch(fh.read())
        if bad:
            raise RuntimeError(f"{src}: scratch accesses inside a loop (kernel, lines, count): {bad}")
    return obj, out


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor
    cc = hipcc()
    jobs = max(1, min(len(SOURCES), len(os.sched_getaffinity(0)), 8))
    with tempfile.TemporaryDirectory(prefix="sage_build_") as tmp:
        with ThreadPoolExecutor(jobs) as pool:
            done = [pool.submit(_compile, cc, tmp, src, extra) for src, extra in SOURCES.items()]
            results = [f.result() for f in done]
        objs = [obj for obj, _ in results]
        if verbose:
            for _, out in results:
                if out.strip():
                    print(out)
        tmp_lib = os.path.join(tmp, "libsage.so")
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs)
        shutil.move(tmp_lib, LIB + ".tmp")
        os.replace(LIB + ".tmp", LIB)
    return LIB

if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
