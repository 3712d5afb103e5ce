"""Python binding of libzeroshard.so (include/zero_shard.h), via ctypes.

Argument marshalling only: tensors are checked for dtype, device and
contiguity and passed as raw device pointers together with torch's current
HIP stream; every step of the shard update runs in the library's kernels.
Importing this module loads the library and fails loudly if it is missing or
was not built for this tree; there is no fallback path.

torch is imported first so that the library binds to the HIP runtime torch
already loaded (both name the same soname, libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import NamedTuple, Optional, Sequence, Tuple

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzeroshard.so")

ZERO_OK = 0
ZERO_EINVAL = -1
ZERO_EOVERFLOW = -2
ZERO_EHIP = -3
ZERO_ENOMEM = -4
ZERO_ENOTSUP = -5
ZERO_ERANGE = -6
ZERO_NOALLOC_SCRATCH_BYTES = 8 << 20
ZERO_NOALLOC_MAX_TENSORS = 1024
ZERO_MAX_SLICES = 256
ZERO_FUSED_SPLIT_SLICES = 16
ZERO_LOG2_SCALE_MAX = 100


class ZeroError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({zero_status_str(status)})")
        self.status = status


class _Layout(ctypes.Structure):
    _fields_ = [("padded_total", ctypes.c_uint64), ("shard_len", ctypes.c_uint64),
                ("offset", ctypes.c_uint64), ("real_len", ctypes.c_uint64)]


class _Comm(ctypes.Structure):
    _fields_ = [("passes", ctypes.c_uint64), ("volume_elems", ctypes.c_uint64),
                ("ring_send_elems", ctypes.c_uint64)]


class _Tensor(ctypes.Structure):
    _fields_ = [("param_f16", ctypes.c_void_p), ("grad_f16", ctypes.c_void_p),
                ("master", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("n", ctypes.c_uint64)]


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


class _OffloadInfo(ctypes.Structure):
    _fields_ = [("threads", ctypes.c_uint32), ("numa_node", ctypes.c_int32),
                ("pinned_cpus", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("chunk_elems", ctypes.c_uint64)]


class _Stats(ctypes.Structure):
    _fields_ = [(k, ctypes.c_uint64) for k in (
        "n_tensors", "n_params", "n_chunks", "chunk_elems", "vector_elems",
        "scalar_elems", "table_bytes", "tile_elems", "wg_per_cu")]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    i32, u32, u64, vp = ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p
    sig = {
        "zero_shard_layout": [u64, u32, u32, u32, ctypes.POINTER(_Layout)],
        "zero_state_bytes": [u32, u64, u32, u32, ctypes.POINTER(ctypes.c_uint64)],
        "zero_comm_volume": [u32, u64, u32, u32, ctypes.POINTER(_Comm)],
        "zero_gather_shards": [ctypes.POINTER(vp), u32, u64, vp, vp],
        "zero_plan_create": [ctypes.POINTER(_Tensor), u32, u32, ctypes.POINTER(vp)],
        "zero_plan_create_bf16": [ctypes.POINTER(_Tensor), u32, u32, ctypes.POINTER(vp)],
        "zero_reduce_grad_shard_bf16": [ctypes.POINTER(vp), u32, u64, vp, vp, vp],
        "zero_plan_stats_of": [vp, ctypes.POINTER(_Stats)],
        "zero_plan_describe": [ctypes.POINTER(_Tensor), u32, u32, ctypes.POINTER(_Stats)],
        "zero_plan_destroy": [vp],
        "zero_adam_scalars": [ctypes.POINTER(_HParams), u64, ctypes.POINTER(ctypes.c_float)],
        "zero_adam_step": [vp, ctypes.POINTER(_HParams), u64, vp, vp, vp],
        "zero_adam_step_scaled": [vp, ctypes.POINTER(_HParams), u64, vp, vp, vp, vp],
        "zero_adam_step_noalloc": [ctypes.POINTER(_Tensor), u32, ctypes.POINTER(_HParams), u64,
                                   vp, vp, vp],
        "zero_loss_scale_update": [vp, vp, u32, ctypes.c_int32, ctypes.c_int32, vp],
        "zero_reduce_grad_shard": [ctypes.POINTER(vp), u32, u64, vp, vp, vp],
        "zero_reduce_adam_step": [ctypes.POINTER(vp), u32, u64, vp, vp, vp, vp, vp,
                                  ctypes.POINTER(_HParams), u64, vp, vp],
        "zero_reduce_adam_step_bf16": [ctypes.POINTER(vp), u32, u64, vp, vp, vp, vp, vp,
                                       ctypes.POINTER(_HParams), u64, vp, vp],
        "zero_adam_step_host": [vp, vp, vp, vp, vp, u64, ctypes.POINTER(_HParams), u64, u32, vp],
        "zero_adam_step_host_bf16": [vp, vp, vp, vp, vp, u64, ctypes.POINTER(_HParams), u64, u32,
                                     vp],
        "zero_offload_create": [u64, u32, ctypes.POINTER(vp)],
        "zero_offload_destroy": [vp],
        "zero_offload_describe": [vp, ctypes.POINTER(_OffloadInfo)],
        "zero_offload_step": [vp, vp, vp, vp, vp, vp, u64, ctypes.POINTER(_HParams), u64, vp, vp],
        "zero_offload_step_bf16": [vp, vp, vp, vp, vp, vp, u64, ctypes.POINTER(_HParams), u64, vp,
                                   vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = i32
    L.zero_status_str.argtypes = [i32]
    L.zero_status_str.restype = ctypes.c_char_p
    return L


_lib = _load()

# Every symbol include/zero_shard.h declares.
EXPORTS = ("zero_shard_layout", "zero_state_bytes", "zero_comm_volume",
           "zero_gather_shards", "zero_plan_create", "zero_plan_create_bf16",
           "zero_reduce_grad_shard_bf16",
           "zero_plan_stats_of", "zero_plan_describe", "zero_plan_destroy",
           "zero_adam_scalars", "zero_adam_step", "zero_reduce_grad_shard",
           "zero_reduce_adam_step", "zero_reduce_adam_step_bf16", "zero_adam_step_host",
           "zero_adam_step_host_bf16", "zero_offload_create", "zero_offload_step_bf16",
           "zero_offload_destroy", "zero_offload_describe", "zero_offload_step", "zero_status_str",
           "zero_adam_step_scaled", "zero_loss_scale_update", "zero_adam_step_noalloc")


def lib() -> ctypes.CDLL:
    return _lib


def zero_status_str(status: int) -> str:
    return _lib.zero_status_str(int(status)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != ZERO_OK:
        raise ZeroError(fn, rc)


class Layout(NamedTuple):
    padded_total: int
    shard_len: int
    offset: int
    real_len: int


def zero_shard_layout(psi: int, nd: int, rank: int, align: int = 1) -> Layout:
    out = _Layout()
    _check("zero_shard_layout", _lib.zero_shard_layout(psi, nd, rank, align, ctypes.byref(out)))
    return Layout(out.padded_total, out.shard_len, out.offset, out.real_len)


def zero_state_bytes(stage: int, psi: int, nd: int, align: int = 1) -> int:
    out = ctypes.c_uint64()
    _check("zero_state_bytes", _lib.zero_state_bytes(stage, psi, nd, align, ctypes.byref(out)))
    return out.value


def zero_comm_volume(stage: int, psi: int, nd: int, align: int = 1) -> dict:
    """Elements one rank moves per step: {passes, volume_elems, ring_send_elems}."""
    out = _Comm()
    _check("zero_comm_volume", _lib.zero_comm_volume(stage, psi, nd, align, ctypes.byref(out)))
    return {k: getattr(out, k) for k, _ in _Comm._fields_}


@dataclass(frozen=True)
class AdamHParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0

    def _c(self) -> _HParams:
        return _HParams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay)


def _hp(hp) -> _HParams:
    if isinstance(hp, dict):
        hp = AdamHParams(**hp)
    return hp._c()


def zero_adam_scalars(hp, t: int) -> Tuple[float, ...]:
    """{lr, b1, 1-b1, b2, 1-b2, 1-b1^t, 1-b2^t, eps} as the kernel uses them."""
    out = (ctypes.c_float * 8)()
    h = _hp(hp)
    _check("zero_adam_scalars", _lib.zero_adam_scalars(ctypes.byref(h), t, out))
    return tuple(out)


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, dtype, what: str, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: expected a device (cuda/HIP) tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{what}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")


def _flag_ptr(flag: Optional[torch.Tensor], what: str, device) -> Optional[int]:
    if flag is None:
        return None
    _need(flag, torch.int32, what, device)
    if flag.numel() < 1:
        raise ValueError(f"{what}: needs one int32")
    return flag.data_ptr()


def _tensor_entries(tensors: Sequence[Sequence[torch.Tensor]], half=torch.float16):
    """half: the 16-bit dtype of every parameter and gradient (float16 or
    bfloat16)."""
    arr = (_Tensor * max(1, len(tensors)))()
    device = None
    for k, group in enumerate(tensors):
        if len(group) != 5:
            raise ValueError("each tensor is (param, grad, master, m, v)")
        p, g, w, m, v = group
        device = device or w.device
        for x, dt, nm in ((p, half, "param"), (g, half, "grad"),
                          (w, torch.float32, "master"), (m, torch.float32, "m"),
                          (v, torch.float32, "v")):
            _need(x, dt, f"tensor {k} {nm}", device)
        n = w.numel()
        if not (p.numel() == g.numel() == m.numel() == v.numel() == n):
            raise ValueError(f"tensor {k}: the five arrays differ in size")
        arr[k] = _Tensor(p.data_ptr(), g.data_ptr(), w.data_ptr(), m.data_ptr(),
                         v.data_ptr(), n)
    return arr, device


class Plan:
    """A zero_plan: the device chunk table over a list of tensors.  Holds
    references to the tensors so their memory outlives the plan."""

    def __init__(self, handle: int, tensors, device):
        self._h = handle
        self._keep = [tuple(g) for g in tensors]
        self.device = device

    @property
    def handle(self) -> int:
        if not self._h:
            raise ValueError("plan was destroyed")
        return self._h

    def stats(self) -> dict:
        s = _Stats()
        _check("zero_plan_stats_of", _lib.zero_plan_stats_of(self.handle, ctypes.byref(s)))
        return {k: getattr(s, k) for k, _ in _Stats._fields_}

    def destroy(self) -> None:
        if self._h:
            h, self._h = self._h, None
            _check("zero_plan_destroy", _lib.zero_plan_destroy(h))
            self._keep = []

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def zero_plan_create(tensors: Sequence[Sequence[torch.Tensor]], chunk_elems: int = 0) -> Plan:
    """tensors: sequence of (param, grad, master_f32, m_f32, v_f32) where
    every param and grad is float16 (the pages' ledger) or every one is
    bfloat16 (the bfloat16 variant).  chunk_elems: 0 for the library
    default, else a multiple of 512."""
    half = tensors[0][0].dtype if len(tensors) else torch.float16
    if half not in (torch.float16, torch.bfloat16):
        raise TypeError(f"param: expected torch.float16 or torch.bfloat16, got {half}")
    arr, device = _tensor_entries(tensors, half)
    fn = "zero_plan_create_bf16" if half == torch.bfloat16 else "zero_plan_create"
    h = ctypes.c_void_p()
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check(fn, getattr(_lib, fn)(arr, len(tensors), int(chunk_elems), ctypes.byref(h)))
    return Plan(h.value, tensors, device)


def zero_plan_describe(tensors, chunk_elems: int = 0) -> dict:
    """Classification of a would-be plan, computed on the host only.
    tensors: sequence of (param, grad, master, m, v, n) with integer
    addresses, or of torch tensors as for zero_plan_create."""
    arr = (_Tensor * max(1, len(tensors)))()
    for k, e in enumerate(tensors):
        if len(e) == 6:
            arr[k] = _Tensor(*e)
        else:
            a, _ = _tensor_entries([e])
            arr[k] = a[0]
    s = _Stats()
    _check("zero_plan_describe", _lib.zero_plan_describe(arr, len(tensors), int(chunk_elems),
                                                         ctypes.byref(s)))
    return {k: getattr(s, k) for k, _ in _Stats._fields_}


def zero_plan_destroy(plan: Plan) -> None:
    plan.destroy()


def zero_adam_step(plan: Plan, hp, t: int, nonfinite_flag: Optional[torch.Tensor] = None,
                   skip_if_nonzero: Optional[torch.Tensor] = None, stream=None,
                   loss_scale: Optional["LossScale"] = None) -> None:
    """Enqueue one Adam step over the plan on `stream` (torch's current stream
    by default).  With `loss_scale`, the gradients carry its factor 2^k and
    are multiplied by 2^-k first (zero_adam_step_scaled)."""
    h = _hp(hp)
    f = _flag_ptr(nonfinite_flag, "nonfinite_flag", plan.device)
    s = _flag_ptr(skip_if_nonzero, "skip_if_nonzero", plan.device)
    if loss_scale is None:
        _check("zero_adam_step", _lib.zero_adam_step(plan.handle, ctypes.byref(h), int(t), f, s,
                                                     _stream_handle(stream)))
        return
    if loss_scale.state.device != plan.device:
        raise ValueError(f"loss_scale: on {loss_scale.state.device}, expected {plan.device}")
    _check("zero_adam_step_scaled",
           _lib.zero_adam_step_scaled(plan.handle, ctypes.byref(h), int(t),
                                      loss_scale.state.data_ptr(), f, s, _stream_handle(stream)))


def zero_adam_step_noalloc(tensors: Sequence[Sequence[torch.Tensor]], hp, t: int,
                           nonfinite_flag: Optional[torch.Tensor] = None,
                           skip_if_nonzero: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue one Adam step over float16 tensors (param, grad, master, m, v)
    without a plan: the library rebuilds the chunk table in its fixed
    per-device array and allocates nothing.  Calls that may overlap on one
    device race for that array."""
    arr, device = _tensor_entries(tensors, torch.float16)
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    h = _hp(hp)
    f = _flag_ptr(nonfinite_flag, "nonfinite_flag", device)
    s = _flag_ptr(skip_if_nonzero, "skip_if_nonzero", device)
    with torch.cuda.device(device):
        _check("zero_adam_step_noalloc",
               _lib.zero_adam_step_noalloc(arr, len(tensors), ctypes.byref(h), int(t), f, s,
                                           _stream_handle(stream)))


class LossScale:
    """A dynamic loss scale 2^k held on the device as the four int32 of
    zero_loss_scale: (log2_scale, good_steps, skipped_steps, applied_steps).

    One step: zero_reduce_grad_shard(..., flag); zero_adam_step(plan, hp, t,
    skip_if_nonzero=flag, loss_scale=ls); ls.update(flag) -- which halves the
    scale after a non-finite gradient, doubles it after `interval` finite
    steps in a row, and clears the flag."""

    def __init__(self, log2_scale: int = 16, interval: int = 2000, min_log2: int = 0,
                 max_log2: int = 24, device=None):
        if not -ZERO_LOG2_SCALE_MAX <= min_log2 <= max_log2 <= ZERO_LOG2_SCALE_MAX:
            raise ValueError("need -100 <= min_log2 <= max_log2 <= 100")
        if interval < 1:
            raise ValueError("interval must be >= 1")
        self.interval, self.min_log2, self.max_log2 = int(interval), int(min_log2), int(max_log2)
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        self.state = torch.tensor([int(log2_scale), 0, 0, 0], dtype=torch.int32, device=device)

    def update(self, nonfinite_flag: torch.Tensor, stream=None) -> None:
        """Enqueue the scale's update from the step's flag (then set to 0)."""
        f = _flag_ptr(nonfinite_flag, "nonfinite_flag", self.state.device)
        _check("zero_loss_scale_update",
               _lib.zero_loss_scale_update(self.state.data_ptr(), f, self.interval,
                                           self.min_log2, self.max_log2, _stream_handle(stream)))

    def read(self) -> tuple:
        """(log2_scale, good_steps, skipped_steps, applied_steps); waits for
        the device."""
        v = self.state.cpu().tolist()
        return (v[0], v[1] & 0xFFFFFFFF, v[2] & 0xFFFFFFFF, v[3] & 0xFFFFFFFF)


def zero_reduce_grad_shard(slices: Sequence[torch.Tensor], out: torch.Tensor,
                           nonfinite_flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """out = mean over ranks of the slices, fp32 sum in rank order, rounded
    to out's format: float16, or bfloat16 (the bfloat16 variant)."""
    half = out.dtype if out.dtype in (torch.float16, torch.bfloat16) else torch.float16
    _need(out, half, "out")
    n = out.numel()
    nd = len(slices)
    if nd == 0 or nd > ZERO_MAX_SLICES:
        raise ValueError(f"need 1..{ZERO_MAX_SLICES} slices, got {nd}")
    ptrs = (ctypes.c_void_p * nd)()
    for r, s in enumerate(slices):
        _need(s, half, f"slice {r}", out.device)
        if s.numel() != n:
            raise ValueError(f"slice {r} has {s.numel()} elements, out has {n}")
        ptrs[r] = s.data_ptr()
    f = _flag_ptr(nonfinite_flag, "nonfinite_flag", out.device)
    fn = "zero_reduce_grad_shard_bf16" if half == torch.bfloat16 else "zero_reduce_grad_shard"
    _check(fn, getattr(_lib, fn)(ptrs, nd, n, out.data_ptr(), f, _stream_handle(stream)))


def zero_reduce_adam_step(slices: Sequence[torch.Tensor], param: torch.Tensor,
                          master: torch.Tensor, m: torch.Tensor, v: torch.Tensor, hp, t: int,
                          grad_out: Optional[torch.Tensor] = None,
                          nonfinite_flag: Optional[torch.Tensor] = None, stream=None) -> None:
    """Reduce the 16-bit slices and apply the Adam step in one pass over a
    flat shard (bit-identical to zero_reduce_grad_shard then
    zero_adam_step).  param, the slices and grad_out are all float16 or all
    bfloat16 (the bfloat16 variant)."""
    _need(master, torch.float32, "master")
    dev = master.device
    n = master.numel()
    half = param.dtype if param.dtype in (torch.float16, torch.bfloat16) else torch.float16
    for x, dt, nm in ((param, half, "param"), (m, torch.float32, "m"),
                      (v, torch.float32, "v")):
        _need(x, dt, nm, dev)
        if x.numel() != n:
            raise ValueError(f"{nm} has {x.numel()} elements, master has {n}")
    nd = len(slices)
    if nd == 0 or nd > ZERO_MAX_SLICES:
        raise ValueError(f"need 1..{ZERO_MAX_SLICES} slices, got {nd}")
    ptrs = (ctypes.c_void_p * nd)()
    for r, s in enumerate(slices):
        _need(s, half, f"slice {r}", dev)
        if s.numel() != n:
            raise ValueError(f"slice {r} has {s.numel()} elements, master has {n}")
        ptrs[r] = s.data_ptr()
    go = None
    if grad_out is not None:
        _need(grad_out, half, "grad_out", dev)
        if grad_out.numel() != n:
            raise ValueError(f"grad_out has {grad_out.numel()} elements, master has {n}")
        go = grad_out.data_ptr()
    h = _hp(hp)
    f = _flag_ptr(nonfinite_flag, "nonfinite_flag", dev)
    name = "zero_reduce_adam_step_bf16" if half == torch.bfloat16 else "zero_reduce_adam_step"
    _check(name, getattr(_lib, name)(ptrs, nd, n, param.data_ptr(), master.data_ptr(),
                                     m.data_ptr(), v.data_ptr(), go, ctypes.byref(h), int(t), f,
                                     _stream_handle(stream)))


def zero_gather_shards(shards: Sequence[torch.Tensor], full: torch.Tensor, stream=None) -> None:
    """full[r * S:(r + 1) * S] = shards[r] for every rank r (fp16); shards
    that are already views at their place in full are left alone."""
    _need(full, torch.float16, "full")
    nd = len(shards)
    if nd == 0 or nd > ZERO_MAX_SLICES:
        raise ValueError(f"need 1..{ZERO_MAX_SLICES} shards, got {nd}")
    S = shards[0].numel()
    if full.numel() != nd * S:
        raise ValueError(f"full has {full.numel()} elements, {nd} shards of {S} need {nd * S}")
    ptrs = (ctypes.c_void_p * nd)()
    for r, s in enumerate(shards):
        _need(s, torch.float16, f"shard {r}", full.device)
        if s.numel() != S:
            raise ValueError(f"shard {r} has {s.numel()} elements, shard 0 has {S}")
        ptrs[r] = s.data_ptr()
    _check("zero_gather_shards",
           _lib.zero_gather_shards(ptrs, nd, S, full.data_ptr(), _stream_handle(stream)))


def _host(a, dtype, what: str, n: Optional[int] = None) -> int:
    """Address of a contiguous host numpy array of the given element type."""
    import numpy as np
    if not isinstance(a, np.ndarray):
        raise TypeError(f"{what}: expected a numpy array")
    if a.dtype.itemsize != np.dtype(dtype).itemsize or a.dtype.kind != np.dtype(dtype).kind:
        if not (np.dtype(dtype) == np.uint16 and a.dtype == np.float16):
            raise TypeError(f"{what}: expected {np.dtype(dtype)}, got {a.dtype}")
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError(f"{what}: must be contiguous")
    if n is not None and a.size != n:
        raise ValueError(f"{what}: has {a.size} elements, expected {n}")
    return a.ctypes.data


def zero_adam_step_host(grad16, param16, master, m, v, hp, t: int, threads: int = 0,
                        nonfinite_flag=None, fmt: str = "f16") -> None:
    """The Adam step on the host CPU over numpy arrays (16-bit values as
    uint16, or float16 for fmt "f16"; fp32 state updated in place);
    bit-identical to zero_adam_step.  fmt: "f16", or "bf16" for the
    bfloat16 variant (gradient and parameter as bfloat16 bit patterns)."""
    if fmt not in ("f16", "bf16"):
        raise ValueError('fmt must be "f16" or "bf16"')
    import numpy as np
    n = master.size
    ptrs = [_host(grad16, np.uint16, "grad", n), _host(param16, np.uint16, "param", n),
            _host(master, np.float32, "master", n), _host(m, np.float32, "m", n),
            _host(v, np.float32, "v", n)]
    f = None if nonfinite_flag is None else _host(nonfinite_flag, np.int32, "nonfinite_flag", 1)
    h = _hp(hp)
    name = "zero_adam_step_host_bf16" if fmt == "bf16" else "zero_adam_step_host"
    _check(name, getattr(_lib, name)(*ptrs, n, ctypes.byref(h), int(t), int(threads), f))


class Offload:
    """A zero_offload pipeline (pinned staging, copy streams, host threads)."""

    def __init__(self, handle: int, device):
        self._h = handle
        self.device = device

    @property
    def handle(self) -> int:
        if not self._h:
            raise ValueError("offload was destroyed")
        return self._h

    def step(self, grad: torch.Tensor, param: torch.Tensor, master, m, v, hp, t: int,
             nonfinite_flag=None, stream=None) -> None:
        """grad, param: device tensors, both float16 or both bfloat16 (the
        bfloat16 variant); master, m, v: host numpy fp32 arrays updated in
        place; nonfinite_flag: None or a numpy int32[1]."""
        import numpy as np
        n = master.size
        half = grad.dtype if grad.dtype in (torch.float16, torch.bfloat16) else torch.float16
        _need(grad, half, "grad", self.device)
        _need(param, half, "param", self.device)
        if grad.numel() != n or param.numel() != n:
            raise ValueError("grad, param and the host state differ in size")
        hs = [_host(master, np.float32, "master", n), _host(m, np.float32, "m", n),
              _host(v, np.float32, "v", n)]
        f = None if nonfinite_flag is None else _host(nonfinite_flag, np.int32, "nonfinite_flag", 1)
        h = _hp(hp)
        name = "zero_offload_step_bf16" if half == torch.bfloat16 else "zero_offload_step"
        _check(name, getattr(_lib, name)(self.handle, grad.data_ptr(), param.data_ptr(), *hs, n,
                                         ctypes.byref(h), int(t), f, _stream_handle(stream)))

    def info(self) -> dict:
        """threads, numa_node (-1: unknown), pinned_cpus (0: not pinned),
        chunk_elems."""
        i = _OffloadInfo()
        _check("zero_offload_describe", _lib.zero_offload_describe(self.handle, ctypes.byref(i)))
        return {k: getattr(i, k) for k, _ in _OffloadInfo._fields_ if k != "reserved"}

    def destroy(self) -> None:
        if self._h:
            h, self._h = self._h, None
            _check("zero_offload_destroy", _lib.zero_offload_destroy(h))

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def zero_offload_create(chunk_elems: int = 0, threads: int = 0) -> Offload:
    h = ctypes.c_void_p()
    _check("zero_offload_create", _lib.zero_offload_create(int(chunk_elems), int(threads),
                                                           ctypes.byref(h)))
    return Offload(h.value, torch.device("cuda", torch.cuda.current_device()))
