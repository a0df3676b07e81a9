"""The C ABI's host-side argument validation, built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (device code is compiled as
usual and never launched), driven by tests/host_sanitize/abi_driver.cpp: every
entry point with null, misaligned, negative, oversized and overflowing
arguments must return its documented error code before any HIP call, with no
sanitizer report.  Runs on the CPU; takes a few tens of seconds to build."""
import concurrent.futures
import os
import shutil
import subprocess
import tempfile

import pytest

from exact_attention_04_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host_sanitize", "abi_driver.cpp")
# sanitizers for the host pass only; the flag order keeps them off the device
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def clangxx():
    p = "/opt/rocm/llvm/bin/clang++"
    return p if os.path.exists(p) else shutil.which("clang++")


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs the ROCm compiler")
def test_abi_validation_under_asan_and_ubsan():
    tmp = tempfile.mkdtemp(prefix="attn_asan_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [B.hipcc(), *B.HIP_FLAGS, *B.FILE_FLAGS.get(src, []), *HOST_SANITIZE, "-x", "hip", "-c",
                   os.path.join(B.CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr}"
            return obj
        with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
            objs = list(ex.map(compile_one, B.SOURCES))
        exe = os.path.join(tmp, "abi_driver")
        cmd = [clangxx(), "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(B.ROOT, "include"), DRIVER, *objs, "-L/opt/rocm/lib", "-lamdhip64",
               "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr}"
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        print(r.stdout[-2000:])
        assert r.returncode == 0, f"driver failed (rc {r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
        assert "0 failures" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
