"""Comparison rules for the HIP path against the oracle, and host<->device
helpers.  The bar:
  fp32 master, m, v: relative error <= 1e-6 where the oracle's value is
    nonzero, equal (either sign of zero) where it is zero, and non-finite
    values in the same places with the same class (NaN, +inf, -inf);
  fp16 (or bfloat16) params and reduced gradients: within 1 ulp, measured
    on an ordered integer image of the bits (+0 and -0 both map to 0),
    non-finite classes matching.
Bit-exact counts are reported next to the bar (the design target is
bit-exact: both sides do the same IEEE operations in the same order).
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

REL_TOL = 1e-6
ULP16_TOL = 1


def to_dev16(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.float16)


def to_dev32(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host16(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host32(t) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().astype(np.float32, copy=False)


def _class32(x):
    c = np.zeros(x.shape, np.int8)
    c[np.isnan(x)] = 1
    c[x == np.inf] = 2
    c[x == -np.inf] = 3
    return c


def check32(got: np.ndarray, ref: np.ndarray, what: str) -> dict:
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    assert got.shape == ref.shape, what
    cg, cr = _class32(got), _class32(ref)
    bad_class = np.flatnonzero(cg != cr)
    assert bad_class.size == 0, f"{what}: non-finite class differs at {bad_class[:8]}"
    fin = cr == 0
    g, r = got[fin].astype(np.float64), ref[fin].astype(np.float64)
    nz = r != 0
    rel = np.abs(g[nz] - r[nz]) / np.abs(r[nz])
    max_rel = float(rel.max()) if rel.size else 0.0
    zero_bad = np.flatnonzero(g[~nz] != 0)
    assert zero_bad.size == 0, f"{what}: oracle zero but got nonzero"
    assert max_rel <= REL_TOL, f"{what}: max relative error {max_rel:.3g} > {REL_TOL}"
    not_exact = int(np.count_nonzero(got.view(np.uint32)[fin] != ref.view(np.uint32)[fin]))
    return dict(max_rel=max_rel, not_bit_exact=not_exact, n=int(got.size))


def _ordered16(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


_FMT16 = {"f16": (0x7C00, 0x03FF), "bf16": (0x7F80, 0x007F)}


def _class16(b, fmt="f16"):
    b = np.asarray(b, np.uint16)
    em, fm = _FMT16[fmt]
    exp_all = (b & em) == em
    frac = (b & fm) != 0
    c = np.zeros(b.shape, np.int8)
    c[exp_all & frac] = 1
    c[exp_all & ~frac & ((b & 0x8000) == 0)] = 2
    c[exp_all & ~frac & ((b & 0x8000) != 0)] = 3
    return c


def check16(got: np.ndarray, ref: np.ndarray, what: str, fmt: str = "f16") -> dict:
    """fmt: "f16" or "bf16", the format of both bit-pattern arrays."""
    got = np.asarray(got).view(np.uint16)
    ref = np.asarray(ref).view(np.uint16)
    assert got.shape == ref.shape, what
    cg, cr = _class16(got, fmt), _class16(ref, fmt)
    bad_class = np.flatnonzero(cg != cr)
    assert bad_class.size == 0, f"{what}: non-finite class differs at {bad_class[:8]}"
    fin = cr == 0
    d = np.abs(_ordered16(got[fin]) - _ordered16(ref[fin]))
    max_ulp = int(d.max()) if d.size else 0
    assert max_ulp <= ULP16_TOL, f"{what}: {max_ulp} fp16 ulps apart"
    not_exact = int(np.count_nonzero(got[fin] != ref[fin]))
    return dict(max_ulp=max_ulp, not_bit_exact=not_exact, n=int(got.size))


def check_whole32(got: np.ndarray, ref: np.ndarray, what: str) -> dict:
    """check32 over whole arrays of any size: the elements whose bits differ
    (NaN payloads among them) are found first and only those go through
    the class and relative-error rules."""
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    assert got.shape == ref.shape, what
    diff = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
    r = check32(got[diff], ref[diff], what) if diff.size else dict(max_rel=0.0, not_bit_exact=0)
    r.update(n=int(got.size), bits_differ=int(diff.size))
    return r


def check_whole16(got: np.ndarray, ref: np.ndarray, what: str, fmt: str = "f16") -> dict:
    """check16 over whole arrays of any size, as check_whole32."""
    got = np.asarray(got).view(np.uint16)
    ref = np.asarray(ref).view(np.uint16)
    assert got.shape == ref.shape, what
    diff = np.flatnonzero(got != ref)
    r = check16(got[diff], ref[diff], what, fmt) if diff.size else dict(max_ulp=0, not_bit_exact=0)
    r.update(n=int(got.size), bits_differ=int(diff.size))
    return r


def host_threads() -> int:
    """Host threads for the oracle: the CPUs this process may use, capped
    by the cgroup's CPU quota (a shared machine's share for one GPU)."""
    n = len(os.sched_getaffinity(0))
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            n = min(n, max(1, int(int(q) / int(per))))
    except (OSError, ValueError):
        pass
    return max(1, n)


def on_windows(fn, n: int) -> int:
    """fn(lo, hi) over 8 windows of [0, n) per host thread; the oracle's C
    calls release the interpreter lock.  Returns the OR of the results."""
    T = host_threads()
    parts = 8 * T
    wins = [(n * i // parts, n * (i + 1) // parts) for i in range(parts)]
    with cf.ThreadPoolExecutor(T) as ex:
        flags = list(ex.map(lambda b: fn(*b), wins))
    return int(any(flags))
