"""Plain scalar CPU oracle for one rank's ZeRO shard step (ctypes loader).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
``cpu_baseline`` leg are the only callers.  The product path (the HIP library
and its Python binding) never imports this package.  The arithmetic lives in
``oracle.c`` next to this file; see its header for the sources it follows.

Arrays are numpy arrays: fp16 values travel as ``uint16`` bit patterns (or
``float16`` views of them), fp32 state as ``float32``.  Every function works
in place on the arrays it is given, like the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
          "-fno-tree-vectorize", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, scalar, no FMA)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    """Load liboracle.so (building it if absent or stale).  The tests that
    plant mistakes in a copy of oracle.c point ZERO_ORACLE_LIB at that copy's
    build to check that the pins catch them."""
    global _lib
    if _lib is None:
        path = os.environ.get("ZERO_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        u64, u32, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        vp = ctypes.c_void_p
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16_array.argtypes = [vp, vp, u64]
        L.orc_f32_to_f16_array.restype = None
        L.orc_f16_to_f32_array.argtypes = [vp, vp, u64]
        L.orc_f16_to_f32_array.restype = None
        L.orc_shard_layout.argtypes = [u64, u32, u32, u32, vp]
        L.orc_shard_layout.restype = i32
        L.orc_state_bytes.argtypes = [u32, u64, u32, u32, vp]
        L.orc_state_bytes.restype = i32
        L.orc_adam_scalars.argtypes = [vp, u64, vp]
        L.orc_adam_scalars.restype = i32
        L.orc_adam_step.argtypes = [u64, vp, vp, vp, vp, vp, vp, u64, i32]
        L.orc_adam_step.restype = i32
        L.orc_reduce.argtypes = [u32, vp, u64, vp]
        L.orc_reduce.restype = i32
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16_array.argtypes = [vp, vp, u64]
        L.orc_f32_to_bf16_array.restype = None
        L.orc_bf16_to_f32_array.argtypes = [vp, vp, u64]
        L.orc_bf16_to_f32_array.restype = None
        L.orc_adam_step_fmt.argtypes = [i32, u64, vp, vp, vp, vp, vp, vp, u64, i32]
        L.orc_adam_step_fmt.restype = i32
        L.orc_adam_step_scaled.argtypes = [i32, u64, vp, vp, vp, vp, vp, vp, u64, ctypes.c_int32,
                                           i32]
        L.orc_adam_step_scaled.restype = i32
        L.orc_reduce_fmt.argtypes = [i32, u32, vp, u64, vp]
        L.orc_reduce_fmt.restype = i32
        L.orc_comm_volume.argtypes = [u32, u64, u32, u32, vp]
        L.orc_comm_volume.restype = i32
        L.orc_gather.argtypes = [u32, vp, u64, vp]
        L.orc_gather.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


class OracleError(RuntimeError):
    pass


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to fp16 bit patterns (uint16), nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen fp16 bit patterns (uint16 or float16 array) to fp32, exactly."""
    h = np.ascontiguousarray(h).view(np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 bit patterns (uint16), nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to fp32, exactly."""
    h = np.ascontiguousarray(h).view(np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_bf16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


def shard_layout(psi: int, nd: int, rank: int, align: int) -> dict:
    out = np.zeros(4, dtype=np.uint64)
    rc = lib().orc_shard_layout(psi, nd, rank, align, _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_shard_layout rc={rc}")
    return dict(zip(("padded_total", "shard_len", "offset", "real_len"),
                    (int(v) for v in out)))


def state_bytes(stage: int, psi: int, nd: int, align: int = 1) -> int:
    out = np.zeros(1, dtype=np.uint64)
    rc = lib().orc_state_bytes(stage, psi, nd, align, _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_state_bytes rc={rc}")
    return int(out[0])


def _hp(lr, beta1, beta2, eps, weight_decay=0.0) -> np.ndarray:
    return np.array([lr, beta1, beta2, eps, weight_decay], dtype=np.float64)


def adam_scalars(lr, beta1, beta2, eps, t, weight_decay=0.0) -> np.ndarray:
    """{lr, b1, 1-b1, b2, 1-b2, 1-b1^t, 1-b2^t, eps} as float32."""
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    out = np.zeros(8, dtype=np.float32)
    rc = lib().orc_adam_scalars(_ptr(hp), t, _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_adam_scalars rc={rc}")
    return out


_FMT = {"f16": 0, "bf16": 1}


def adam_step(grad16, param16, master, m, v, *, lr, beta1, beta2, eps, t,
              weight_decay=0.0, skip=False, fmt="f16") -> int:
    """One Adam step in place over this shard; returns the non-finite flag.
    fmt: "f16" (the pages' ledger) or "bf16": the format of the 16-bit
    gradient and parameter bit patterns (uint16 arrays)."""
    n = master.size
    g = np.ascontiguousarray(grad16).view(np.uint16)
    for a, dt in ((param16, np.uint16), (master, np.float32), (m, np.float32),
                  (v, np.float32)):
        assert a.dtype.itemsize == np.dtype(dt).itemsize and a.size == n
    assert g.size == n
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    if fmt == "f16":
        rc = lib().orc_adam_step(n, _ptr(g), _ptr(param16), _ptr(master), _ptr(m),
                                 _ptr(v), _ptr(hp), t, int(bool(skip)))
    else:
        rc = lib().orc_adam_step_fmt(_FMT[fmt], n, _ptr(g), _ptr(param16), _ptr(master),
                                     _ptr(m), _ptr(v), _ptr(hp), t, int(bool(skip)))
    if rc < 0:
        raise OracleError(f"orc_adam_step rc={rc}")
    return rc


def adam_step_scaled(grad16, param16, master, m, v, *, lr, beta1, beta2, eps, t,
                     log2_scale, weight_decay=0.0, skip=False, fmt="f16") -> int:
    """adam_step on gradients that carry a loss scale of 2^log2_scale: each
    widened gradient is multiplied by 2^-log2_scale first (|log2_scale| <=
    100).  Returns the non-finite flag of the gradients after 2^-log2_scale
    (a finite bfloat16 value can overflow fp32 there when log2_scale < 0)."""
    n = master.size
    g = np.ascontiguousarray(grad16).view(np.uint16)
    for a, dt in ((param16, np.uint16), (master, np.float32), (m, np.float32),
                  (v, np.float32)):
        assert a.dtype.itemsize == np.dtype(dt).itemsize and a.size == n
    assert g.size == n
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    rc = lib().orc_adam_step_scaled(_FMT[fmt], n, _ptr(g), _ptr(param16), _ptr(master), _ptr(m),
                                    _ptr(v), _ptr(hp), t, int(log2_scale), int(bool(skip)))
    if rc < 0:
        raise OracleError(f"orc_adam_step_scaled rc={rc}")
    return rc


def loss_scale_update(state, flag, *, interval, min_log2, max_log2):
    """One update of a dynamic loss scale after a step whose gradients had
    the non-finite flag ``flag``.  ``state`` = (log2_scale, good_steps,
    skipped_steps, applied_steps); returns the new tuple.

    Not on the pages (a reading): a step with a non-finite gradient is
    skipped and the scale halves, down to 2^min_log2; every ``interval``-th
    finite step in a row doubles it, up to 2^max_log2, and restarts the
    count.  Powers of two keep the unscaling multiply exact."""
    k, good, skipped, applied = state
    if flag:
        return (max(min_log2, k - 1), 0, skipped + 1, applied)
    good += 1
    if good >= interval:
        return (min(max_log2, k + 1), 0, skipped, applied + 1)
    return (k, good, skipped, applied + 1)


def reduce_grad(slices, out=None, fmt="f16"):
    """Average N_d 16-bit slices (fmt "f16" or "bf16") into the same format;
    returns (out, flag)."""
    arrs = [np.ascontiguousarray(s).view(np.uint16) for s in slices]
    nd = len(arrs)
    n = arrs[0].size if nd else 0
    assert all(a.size == n for a in arrs)
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    ptrs = (ctypes.c_void_p * max(nd, 1))(*[_ptr(a) for a in arrs])
    if fmt == "f16":
        rc = lib().orc_reduce(nd, ctypes.cast(ptrs, ctypes.c_void_p), n, _ptr(out))
    else:
        rc = lib().orc_reduce_fmt(_FMT[fmt], nd, ctypes.cast(ptrs, ctypes.c_void_p), n, _ptr(out))
    if rc < 0:
        raise OracleError(f"orc_reduce rc={rc}")
    return out, rc


def comm_volume(stage: int, psi: int, nd: int, align: int = 1) -> dict:
    """Per-rank communication of one step: {passes, volume, ring_send}, in
    elements (fp16: 2 bytes each)."""
    out = np.zeros(3, dtype=np.uint64)
    rc = lib().orc_comm_volume(stage, psi, nd, align, _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_comm_volume rc={rc}")
    return dict(zip(("passes", "volume", "ring_send"), (int(v) for v in out)))


def gather(shards) -> np.ndarray:
    """Concatenate N_d fp16 shards of equal length into the full buffer."""
    arrs = [np.ascontiguousarray(s).view(np.uint16) for s in shards]
    nd = len(arrs)
    n = arrs[0].size if nd else 0
    assert all(a.size == n for a in arrs)
    out = np.empty(nd * n, dtype=np.uint16)
    ptrs = (ctypes.c_void_p * max(nd, 1))(*[_ptr(a) for a in arrs])
    rc = lib().orc_gather(nd, ctypes.cast(ptrs, ctypes.c_void_p), n, _ptr(out))
    if rc != 0:
        raise OracleError(f"orc_gather rc={rc}")
    return out
