"""The library's host code (zs_host.cpp, zs_offload.cpp) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer and driven over
ragged and invalid inputs by host_sanitize.cpp: layouts and ledgers over a
brute-force range, plan classification of random tensor lists at every
alignment class, the step scalars, and the host Adam step at ragged sizes
and thread counts.  No device calls (the HIP runtime is linked, not used)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_partitioned_mixed_layout_amd", "csrc")


def test_host_code_under_sanitizers(tmp_path):
    if shutil.which("g++") is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("needs g++ and the HIP runtime library")
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "host_sanitize.cpp"),
           os.path.join(CSRC, "zs_host.cpp"), os.path.join(CSRC, "zs_offload.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lpthread", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "0 failures" in r.stdout
