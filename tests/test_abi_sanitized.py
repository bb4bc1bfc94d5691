"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer.

sage_api.cpp and layout.cpp are compiled for the host with g++
-fsanitize=address,undefined, linked with stand-ins for the kernel launchers
(tests/host/launch_stubs.cpp), and tests/test_abi.py runs against that library
in a child process with the sanitizer runtime preloaded.  Any report (heap or
stack overflow, use after free, signed overflow, misaligned access ...) fails
the child and this test.  No GPU is used."""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_attention_sage_amd", "csrc")


def _libasan():
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_logic_under_sanitizers():
    asan = _libasan()
    assert asan, "g++ has no AddressSanitizer runtime"
    with tempfile.TemporaryDirectory(prefix="sage_asan_") as tmp:
        flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-fvisibility=hidden", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
                 "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
        objs = []
        for src in (os.path.join(CSRC, "sage_api.cpp"), os.path.join(CSRC, "layout.cpp"),
                    os.path.join(ROOT, "tests", "host", "launch_stubs.cpp")):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            subprocess.run(["g++"] + flags + ["-c", src, "-o", obj], check=True)
            objs.append(obj)
        lib = os.path.join(tmp, "libsage_asan.so")
        subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, "the library is not instrumented"
        env = dict(os.environ, LD_PRELOAD=asan, SAGE_LIBRARY=lib,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_abi.py")], env=env, cwd=ROOT,
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
        assert "passed" in r.stdout and "failed" not in r.stdout
        assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
