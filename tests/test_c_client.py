"""The C ABI from plain C: tests/c_client/host_calls.c includes
include/sfi.h, is compiled by gcc as C99 and linked against libsfi.so, and
runs the calls that need no GPU.  Its scheduler output must equal the
oracle's span schedule for the same seeds."""
import os
import shutil
import subprocess

import pytest

import oracle as O
import sparse_kv_attention_sfi_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is required")
def test_c99_client_of_the_abi(tmp_path):
    lib = S.lib()                                   # builds nothing; fails loudly if the library is missing
    libdir = os.path.dirname(lib._name)
    exe = str(tmp_path / "host_calls")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_client", "host_calls.c"), "-L", libdir, "-lsfi",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c client ok" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])
    steps = [line.split()[3:] for line in r.stdout.splitlines() if line.startswith("step ")]
    assert len(steps) == 64
    flags = [O.schedule("geometric", 18.0, 7 + b, 64) for b in range(3)]
    for t, slow in enumerate(steps):
        assert [int(x) for x in slow] == [b for b in range(3) if flags[b][t]], t
