"""Seeded synthetic inputs for the shard step: shapes, sizes and random draws.

This module holds no arithmetic of the method.  It only says how big the
workloads are and draws their random inputs, so that the HIP path and the CPU
oracle can be fed the same bytes.  Host draws use numpy's Philox generator;
device draws use torch's CUDA generator (followed by torch's own fp32->fp16
cast).  Nothing here imports the HIP library or the oracle.

Workloads (their shapes follow the models the pages use as examples: GPT-2's
largest 1.5B configuration and a 7B model):

  tiny_flat     Psi = 2^20 flat, N_d = 4, rank 0 (262,144 elements), 10 steps,
                with a 1% fp16-underflow gradient set and a 1% swamping set
  gpt2_xl       GPT-2-XL tensor list (580 tensors, 1,557,611,200 params), N_d=1
  flat_7p5b_nd64  Psi = 7.5e9 flat, N_d = 64: 64 fp16 gradient slices of this
                rank's 117,187,500-element partition, reduce then Adam
  flat_7p5b_nd8   Psi = 7.5e9 flat, N_d = 8, rank 3, align 512
                (937,500,160 elements), 0.01% infinite gradients at the timed step
  llama_7b      Llama-7B tensor list (291 tensors, 6,738,415,616 params), N_d=1
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

ADAM_HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
MASTER_STD = 0.02
GRAD_STD = 1e-3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    psi: int
    nd: int
    rank: int
    align: int
    seed: int
    tensors: Tuple[Tuple[str, int], ...]   # (name, numel); flat workloads: one
    warm_steps: int = 0                      # Adam steps before the measured one
    steps: int = 1                           # measured steps (tiny_flat: 10)
    underflow_frac: float = 0.0              # tiny_flat only
    swamp_frac: float = 0.0                  # tiny_flat only
    inf_frac: float = 0.0                    # flat_7p5b_nd8 only
    reduce_slices: bool = False              # flat_7p5b_nd64 only

    @property
    def n_params(self) -> int:
        return sum(n for _, n in self.tensors)


def gpt2_xl_tensors(layers=48, d=1600, vocab=50257, ctx=1024):
    """GPT-2-XL parameter list: biases, LayerNorm weight+bias, tied LM head."""
    out = [("wte", vocab * d), ("wpe", ctx * d)]
    for i in range(layers):
        p = f"h{i}."
        out += [(p + "ln_1.w", d), (p + "ln_1.b", d),
                (p + "attn.c_attn.w", d * 3 * d), (p + "attn.c_attn.b", 3 * d),
                (p + "attn.c_proj.w", d * d), (p + "attn.c_proj.b", d),
                (p + "ln_2.w", d), (p + "ln_2.b", d),
                (p + "mlp.c_fc.w", d * 4 * d), (p + "mlp.c_fc.b", 4 * d),
                (p + "mlp.c_proj.w", 4 * d * d), (p + "mlp.c_proj.b", d)]
    out += [("ln_f.w", d), ("ln_f.b", d)]
    return tuple(out)


def llama_7b_tensors(layers=32, d=4096, ffn=11008, vocab=32000):
    """Llama-7B parameter list: no biases, RMSNorm vectors, untied head."""
    out = [("embed", vocab * d)]
    for i in range(layers):
        p = f"l{i}."
        out += [(p + "q", d * d), (p + "k", d * d), (p + "v", d * d),
                (p + "o", d * d), (p + "gate", d * ffn), (p + "up", d * ffn),
                (p + "down", ffn * d), (p + "attn_norm", d), (p + "ffn_norm", d)]
    out += [("norm", d), ("lm_head", vocab * d)]
    return tuple(out)


def _flat(name, psi, nd, rank, align):
    """One flat tensor holding this rank's real shard length (tail padding
    excluded); the length is the workload's, written out, not computed."""
    return ((name, _REAL_LEN[(psi, nd, rank, align)]),)


# Real shard lengths of the flat workloads (ceil(Psi / (N_d*align)) * align,
# clipped to Psi), written out as data so this module carries no layout code.
_REAL_LEN = {
    (2 ** 20, 4, 0, 1): 262_144,
    (7_500_000_000, 64, 0, 1): 117_187_500,
    (7_500_000_000, 8, 3, 512): 937_500_160,
}

WORKLOADS = {
    "tiny_flat": Workload("tiny_flat", 2 ** 20, 4, 0, 1, 1001,
                          _flat("flat", 2 ** 20, 4, 0, 1), warm_steps=0, steps=10,
                          underflow_frac=0.01, swamp_frac=0.01),
    "gpt2_xl": Workload("gpt2_xl", 1_557_611_200, 1, 0, 1, 1002,
                        gpt2_xl_tensors(), warm_steps=5),
    "flat_7p5b_nd64": Workload("flat_7p5b_nd64", 7_500_000_000, 64, 0, 1, 1003,
                               _flat("flat", 7_500_000_000, 64, 0, 1),
                               reduce_slices=True),
    "flat_7p5b_nd8": Workload("flat_7p5b_nd8", 7_500_000_000, 8, 3, 512, 1004,
                              _flat("flat", 7_500_000_000, 8, 3, 512),
                              warm_steps=5, inf_frac=1e-4),
    "llama_7b": Workload("llama_7b", 6_738_415_616, 1, 0, 1, 1005,
                         llama_7b_tensors(), warm_steps=5),
}


# ---------------------------------------------------------------------------
# Seeds.  Step-t gradients use seed*100 + t, slice r uses seed*1000 + r,
# tensor k of a list offsets those by 7919*k.
# ---------------------------------------------------------------------------
def grad_seed(seed: int, t: int, tensor: int = 0) -> int:
    return seed * 100 + t + 7919 * tensor


def master_seed(seed: int, tensor: int = 0) -> int:
    return seed * 10 + 7919 * tensor + 3


def slice_seed(seed: int, r: int) -> int:
    return seed * 1000 + r


# ---------------------------------------------------------------------------
# Host (numpy) draws: exact and reproducible without a GPU.
# ---------------------------------------------------------------------------
def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(seed))


def host_master(n: int, seed: int, std: float = MASTER_STD) -> np.ndarray:
    return (_rng(seed).standard_normal(n) * std).astype(np.float32)


def host_grad16(n: int, seed: int, std: float = GRAD_STD) -> np.ndarray:
    """fp16 gradients ~ N(0, std), as a float16 array (numpy's RNE cast)."""
    return (_rng(seed).standard_normal(n) * std).astype(np.float16)


def tiny_special_sets(n: int, seed: int, underflow_frac: float,
                      swamp_frac: float) -> Tuple[np.ndarray, np.ndarray]:
    """Disjoint, fixed index sets: (underflow gradients, swamped masters)."""
    k_u = int(round(n * underflow_frac))
    k_s = int(round(n * swamp_frac))
    idx = _rng(seed + 17).permutation(n)
    return np.sort(idx[:k_u]), np.sort(idx[k_u:k_u + k_s])


def tiny_initial_state(wl: Workload):
    """master, m, v, fp16 param for the tiny flat shard.  The swamping set
    gets |master| in [8, 16); m = v = 0; the fp16 param starts as the
    fp16 cast of the master (numpy RNE)."""
    n = wl.n_params
    master = host_master(n, master_seed(wl.seed))
    under, swamp = tiny_special_sets(n, wl.seed, wl.underflow_frac, wl.swamp_frac)
    r = _rng(wl.seed + 29)
    mag = r.uniform(8.0, 16.0, swamp.size)
    sign = np.where(r.random(swamp.size) < 0.5, -1.0, 1.0)
    master[swamp] = (sign * mag).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    param16 = master.astype(np.float16)
    return master, m, v, param16


def tiny_grad16(wl: Workload, t: int) -> np.ndarray:
    """Step-t fp16 gradients for the tiny shard: N(0, 1e-3) except the
    underflow set, which draws sign * U(0, 2^-24) (so its fp16 values are
    +-0 or +-2^-24)."""
    n = wl.n_params
    g = (_rng(grad_seed(wl.seed, t)).standard_normal(n) * GRAD_STD)
    under, _ = tiny_special_sets(n, wl.seed, wl.underflow_frac, wl.swamp_frac)
    r = _rng(grad_seed(wl.seed, t) + 31)
    tiny = r.uniform(0.0, 2.0 ** -24, under.size)
    sign = np.where(r.random(under.size) < 0.5, -1.0, 1.0)
    g[under] = sign * tiny
    return g.astype(np.float16)


def inf_positions(n: int, frac: float, seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """Sorted distinct positions and signs (+1/-1) of injected infinities."""
    k = int(n * frac)
    r = _rng(seed + 41)
    pos = np.sort(r.choice(n, size=k, replace=False, shuffle=False))
    sign = np.where(r.random(k) < 0.5, -1, 1).astype(np.int8)
    return pos.astype(np.int64), sign


# ---------------------------------------------------------------------------
# Device (torch) draws for the large workloads.
# ---------------------------------------------------------------------------
def device_normal(n: int, std: float, seed: int, dtype, device="cuda",
                  out=None):
    """N(0, std) draw on the device, cast by torch to `dtype` (fp16: RNE).
    Drawn in pieces of at most 2^28 elements to bound the fp32 temporary;
    each piece has its own generator seeded from (seed, piece)."""
    import torch
    if out is None:
        out = torch.empty(n, dtype=dtype, device=device)
    piece = 1 << 28
    g = torch.Generator(device=device)
    for k, s in enumerate(range(0, n, piece)):
        e = min(n, s + piece)
        g.manual_seed(seed * 4099 + k)
        tmp = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        tmp.mul_(std)
        out[s:e].copy_(tmp)
        del tmp
    return out


def sample_indices(n: int, k: int, seed: int, must: Optional[np.ndarray] = None,
                   edges: bool = True) -> np.ndarray:
    """k distinct random indices in [0, n) plus both ends, plus `must`."""
    k = min(k, n)
    r = _rng(seed + 53)
    idx = r.choice(n, size=k, replace=False, shuffle=False) if k else np.zeros(0, np.int64)
    parts = [idx.astype(np.int64)]
    if edges and n:
        e = np.arange(min(n, 4096), dtype=np.int64)
        parts += [e, n - 1 - e]
    if must is not None:
        parts.append(np.asarray(must, dtype=np.int64))
    return np.unique(np.concatenate(parts))


# ---------------------------------------------------------------------------
# Device state for the large workloads.  Sizes and offsets come from the
# caller (the shard layout is not computed here).
# ---------------------------------------------------------------------------
class DeviceTensor:
    """The five arrays of one tensor of the shard, on the device.  half: the
    16-bit dtype of the parameter and gradient (torch.float16 by default;
    torch.bfloat16 for the bfloat16 variant)."""

    def __init__(self, n: int, device, param=None, half=None, views=None):
        import torch
        half = half or torch.float16
        self.n = n
        if views is not None:                 # five existing arrays of n elements
            self.p, self.g, self.w, self.m, self.v = views
            return
        self.p = param if param is not None else torch.zeros(n, dtype=half, device=device)
        self.g = torch.zeros(n, dtype=half, device=device)
        self.w = torch.empty(n, dtype=torch.float32, device=device)
        self.m = torch.zeros(n, dtype=torch.float32, device=device)
        self.v = torch.zeros(n, dtype=torch.float32, device=device)

    def arrays(self):
        return (self.p, self.g, self.w, self.m, self.v)


LIST_LAYOUTS = ("flat", "separate")


def device_list_state(wl: Workload, device="cuda", half=None,
                      layout="flat") -> List[DeviceTensor]:
    """One DeviceTensor per tensor of a list workload; master ~ N(0, 0.02).

    layout "flat": the flattened state a ZeRO rank holds -- five buffers of
    n_params elements (fp16 parameters, fp16 gradients, fp32 master, m, v),
    each tensor a view at its running offset, in list order.
    layout "separate": five allocations per tensor, in the order p, g, w, m,
    v, as a model that owns its parameters one tensor at a time holds them.
    Both draw the same values from the same seeds."""
    import torch
    if layout not in LIST_LAYOUTS:
        raise ValueError(f"layout must be one of {LIST_LAYOUTS}")
    half = half or torch.float16
    bufs = None
    if layout == "flat":
        total = wl.n_params
        bufs = [torch.zeros(total, dtype=dt, device=device)
                for dt in (half, half, torch.float32, torch.float32, torch.float32)]
    out, off = [], 0
    for k, (_, n) in enumerate(wl.tensors):
        if bufs is None:
            t = DeviceTensor(n, device, half=half)
        else:
            t = DeviceTensor(n, device, half=half, views=[b[off:off + n] for b in bufs])
            off += n
        device_normal(n, MASTER_STD, master_seed(wl.seed, k), None, device, out=t.w)
        out.append(t)
    return out


def device_flat_state(wl: Workload, offset: int, length: int, padded_total: int,
                      device="cuda", half=None):
    """The flat workloads: the full fp16 parameter buffer of padded_total
    elements (every rank holds all fp16 parameters under stages 1-2) and this
    rank's shard of `length` elements at `offset` in it.  Returns
    (param_full, DeviceTensor)."""
    import torch
    full = torch.zeros(padded_total, dtype=half or torch.float16, device=device)
    t = DeviceTensor(length, device, param=full[offset:offset + length], half=half)
    device_normal(length, MASTER_STD, master_seed(wl.seed), None, device, out=t.w)
    return full, t


def device_fill_grads(wl: Workload, tensors: Sequence[DeviceTensor], t: int) -> None:
    """Step-t fp16 gradients ~ N(0, 1e-3) for every tensor, in place."""
    for k, dt in enumerate(tensors):
        device_normal(dt.n, GRAD_STD, grad_seed(wl.seed, t, k), None, dt.g.device, out=dt.g)


def device_inject_inf(grad, positions: np.ndarray, signs: np.ndarray) -> None:
    """Set grad[positions] to +inf or -inf (fp16)."""
    import torch
    pos = torch.from_numpy(positions).to(grad.device)
    val = torch.from_numpy(signs.astype(np.float32) * np.float32(np.inf)).to(grad.device)
    grad.index_copy_(0, pos, val.to(grad.dtype))


def device_slices(wl: Workload, length: int, device="cuda", half=None, back_to_back=False):
    """N_d fp16 gradient slices of this rank's partition, ~ N(0, 1e-3), as
    rows of one buffer whose row pitch is rounded up to 64 elements (so every
    row starts 128-byte aligned, as separately allocated receive buffers
    would), or with back_to_back at r * length in one buffer (a receive
    buffer of N_d shards).  Returns (buffer, [row views])."""
    import torch
    pitch = length if back_to_back else (length + 63) // 64 * 64
    buf = torch.zeros(wl.nd, pitch, dtype=half or torch.float16, device=device)
    rows = [buf[r, :length] for r in range(wl.nd)]
    for r in range(wl.nd):
        device_normal(length, GRAD_STD, slice_seed(wl.seed, r), None, device, out=rows[r])
    return buf, rows
