"""One data-parallel rank's ZeRO partition step for mixed-precision Adam on
AMD MI355X (gfx950).

The compute lives in libzeroshard.so (C ABI: include/zero_shard.h, HIP
kernels in csrc/).  Submodules:
  zero_shard  the Python binding; importing it loads the library and raises
              ImportError if it is not built (there is no fallback path)
  workloads   seeded synthetic inputs (shapes and random draws only)
  build       compiles the library with hipcc for gfx950
"""
