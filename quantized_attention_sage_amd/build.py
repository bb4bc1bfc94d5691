"""Build libsage.so (HIP kernels for gfx950 + the C ABI) in the package folder.

    python -m quantized_attention_sage_amd.build

Every source is compiled with hipcc for gfx950 only.  The quantisation
kernels are compiled without floating-point contraction (their fp32 results
decide integer and FP8 codes and must be exactly reproducible).

The attention kernels wait for their own global-to-LDS copies by count
(s_waitcnt vmcnt).  A register spill inside their key loop would add compiler
memory operations to those counts (which only makes the waits stricter, but
costs a full wait for every reload), so the build reads the gfx950 assembly of
each attention source and fails if a scratch access sits inside a loop, or
if compiler-generated code uses m0 (which the copies' inline assembly sets).
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
LOOP_SPILL_FREE = ("attn.hip", "attn_pvh.hip", "attn_fp4.hip", "attn_bwd.hip")
SOURCES = {
    "quant.hip": ["-ffp-contract=off"],
    "attn.hip": [],
    "attn_pvh.hip": [],
    "attn_fp4.hip": [],
    "probe.hip": [],
    "static_ws.hip": [],
    "attn_bwd.hip": [],
    "sage_api.cpp": ["-x", "hip"],
    "layout.cpp": ["-x", "hip"],
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
    """(kernel, block label, first line, scratch ops) of every basic block, of
    every kernel in a gfx950 assembly listing, that holds a scratch access and
    lies on a cycle of the kernel's control-flow graph (can reach itself)."""
    bad = []
    lines = asm.splitlines()
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):", lines[i])
        if not m:
            i += 1
            continue
        func, start = m.group(1), i + 1
        end = start
        while end < len(lines) and not lines[end].startswith(".Lfunc_end"):
            end += 1
        # basic blocks: one starts at the entry, at every label and after every branch
        heads = [start]
        for j in range(start, end):
            if re.match(r"^\.LBB\S+:", lines[j]) and heads[-1] != j:
                heads.append(j)
            elif re.match(r"^\s+s_(branch|cbranch_\w+)\s", lines[j]) and j + 1 < end:
                heads.append(j + 1)
        heads = sorted(set(heads))
        names = [lines[h].split(":")[0] if re.match(r"^\.LBB\S+:", lines[h]) else f"<line {h + 1}>" for h in heads]
        index = {n: k for k, n in enumerate(names) if n.startswith(".LBB")}
        succ, scratch = [], []
        for k, h in enumerate(heads):
            stop = heads[k + 1] if k + 1 < len(heads) else end
            out, falls, n_scr = set(), True, 0
            for j in range(h, stop):
                ln = lines[j]
                br = re.match(r"^\s+s_(branch|cbranch_\w+)\s+(\.LBB\S+)", ln)
                if br:
                    out.add(index[br.group(2)])
                    falls = br.group(1) != "branch"
                elif re.match(r"^\s+s_(endpgm|setpc_b64|trap)\b", ln):
                    falls = False
                elif re.match(r"^\s+scratch_", ln):
                    n_scr += 1
            if falls and k + 1 < len(heads):
                out.add(k + 1)
            succ.append(out)
            scratch.append(n_scr)
        for k, n_scr in enumerate(scratch):
            if not n_scr:
                continue
            seen, todo = set(), list(succ[k])
            while todo:
                x = todo.pop()
                if x in seen:
                    continue
                seen.add(x)
                todo.extend(succ[x])
            if k in seen:
                bad.append((func, names[k], heads[k] + 1, n_scr))
        i = end
    return bad


def m0_outside_inline_asm(asm: str) -> list:
    """Line numbers where compiler-generated code names m0.  The attention
    kernels set m0 inside their own inline assembly (global-to-LDS copies);
    m0 is a reserved register for the compiler, so those kernels must hold no
    compiler use of it that an inline copy could overwrite."""
    bad, inside = [], False
    for i, line in enumerate(asm.splitlines()):
        if ";;#ASMSTART" in line:
            inside = True
        elif ";;#ASMEND" in line:
            inside = False
        elif not inside and re.search(r"\bm0\b", line.split(";")[0]):
            bad.append(i + 1)
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
            asm = fh.read()
        bad = loops_with_scratch(asm)
        if bad:
            raise RuntimeError(f"{src}: scratch accesses inside a loop (kernel, block, line, count): {bad}")
        m0 = m0_outside_inline_asm(asm)
        if m0:
            raise RuntimeError(f"{src}: compiler-generated uses of m0 at lines {m0[:10]}")
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
