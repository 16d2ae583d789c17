"""The library's host code (C ABI validation, launch planning, workspace
layout, scheduler, timing registry) built with AddressSanitizer and
UndefinedBehaviorSanitizer for the host only, and driven through every
entry point's host paths by tests/host_sanitize/driver.cpp.  No GPU is
used: the kernel launchers are stubs the driver never reaches."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_kv_attention_sfi_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
HIPCC = "/opt/rocm/bin/hipcc"

# sanitizers for the host side only (each -fsanitize behind -Xarch_host)
COMPILE = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include")]
LINK = ["--offload-arch=gfx950", "-fsanitize=address", "-fsanitize=undefined", "-fno-gpu-sanitize"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is required for the host build")
def test_host_code_under_asan_and_ubsan(tmp_path):
    sources = [os.path.join(CSRC, "sfi_api.cpp"), os.path.join(CSRC, "sfi_sched.cpp"),
               os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *COMPILE, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, sources))
    exe = str(tmp_path / "driver")
    r = subprocess.run([HIPCC, *LINK, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("SFI_FAULT_INJECT", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host checks passed" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
