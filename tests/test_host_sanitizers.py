"""The library's host code (argument validation, planning, status and error
plumbing) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host side only, driven by a C program that calls every entry point with
rejected arguments (tests/host/abi_check.c). No GPU is used: every checked
call returns before anything is enqueued, so the device code, compiled as
usual, never runs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hybrid_precision_quantized_amd", "csrc")
SOURCES = ["hq_api.cpp", "hq_quantize.hip", "hq_decode.hip", "hq_detect.hip", "hq_prefill.hip",
           "hq_stream.hip", "hq_lifecycle.hip"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs = []
    procs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [hipcc, "-x", "hip", *common, *san, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for cmd, p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, " ".join(cmd) + "\n" + out
    drv = str(tmp_path / "abi_check.o")
    r = subprocess.run(["clang", "-O1", "-g", "-fsanitize=address,undefined", "-I", os.path.join(ROOT, "include"),
                        "-c", os.path.join(ROOT, "tests", "host", "abi_check.c"), "-o", drv],
                       capture_output=True, text=True) if shutil.which("clang") else None
    if r is None or r.returncode != 0:
        r = subprocess.run(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fsanitize=address,undefined", "-I",
                            os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "host", "abi_check.c"),
                            "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    exe = str(tmp_path / "abi_check")
    r = subprocess.run([hipcc, "-fsanitize=address,undefined", "--offload-arch=gfx950", drv, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ALL_OK" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
