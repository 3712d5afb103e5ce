"""Build libzeroshard.so (the HIP library behind include/zero_shard.h).

hipcc cross-compiles for gfx950 (MI355X) without a GPU.  Flags that the
library's exactness depends on:
  -ffp-contract=off                       no fused multiply-add in the step
  -fno-gpu-flush-denormals-to-zero        keep fp32 denormals
  -fhip-fp32-correctly-rounded-divide-sqrt IEEE fp32 division and sqrt
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                          no packed fp32 instructions
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzeroshard.so")
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("zs_host.cpp", "zs_kernels.hip", "zs_offload.cpp")]
HEADERS = [os.path.join(ROOT, "include", "zero_shard.h"),
           os.path.join(HERE, "csrc", "zs_internal.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile the library in place (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
