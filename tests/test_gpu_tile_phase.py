"""GPU parity of the Adam step's peeled head (through the C ABI) against the
CPU oracle.  Every array is carved out of a flattened buffer that starts on
a 1 KiB boundary, each tensor in a slot of its own (a multiple of 256
elements) at a chosen element offset o.  The fp32 master, m and v then
reach their next 1 KiB boundary together, (256 - o mod 256) mod 256
elements in, and on a tensor of 1,024 elements or more the head runs up
to there (the first (4 - o mod 4) mod 4 singly, the rest by fours), so
that the tensor's tiles start on 1 KiB of fp32; a smaller tensor, or one
whose v is shifted four elements against master and m (the three then
disagree), keeps only the vector's head.  Offsets give head lengths
from 1 to 255; sizes sit around the head and the tile and chunk
boundaries after it; every element compared, for fp16 and bfloat16 and
for gradients that carry a loss scale.  Each case prints its name and
sizes before it touches the GPU."""
import numpy as np
import pytest

import oracle
from parity import check16, check32, host16, host32, to_dev16, to_dev32
from zero_partitioned_mixed_layout_amd import workloads as W

pytestmark = pytest.mark.gpu
HP = dict(W.ADAM_HP)
KIB = 1024
OFFSETS = [0, 1, 2, 3, 4, 64, 131, 192, 253, 255]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def zs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from zero_partitioned_mixed_layout_amd import zero_shard
    torch.cuda.set_device(0)
    return zero_shard


def _head(o, v_shift, n=1 << 20):
    """The head a tensor of n elements at offset o gets: to the 1 KiB
    boundary from 1,024 elements on when master, m and v agree, else the
    vector head."""
    vec = (4 - o % 4) % 4
    return vec if v_shift or n < 1024 else (256 - o % 256) % 256


def _sizes(h):
    s = {1, 2, 3, 5, 8, h - 1, h, h + 1, h + 3, h + 4, h + 255, h + 256, h + 257,
         h + 513, 1023, 1024, 1025, h + 1024, h + 1025, h + 16383, h + 16389, 70001}
    return sorted(x for x in s if x > 0)


def _aligned(torch, elems, dtype):
    """A device buffer of `elems` elements whose first sits on 1 KiB."""
    size = 2 if dtype == torch.float16 else 4
    raw = torch.zeros(elems + KIB // size, dtype=dtype, device="cuda")
    skip = ((-raw.data_ptr()) % KIB) // size
    return raw[skip:skip + elems]


class Carved:
    """Five flattened buffers holding (offset, n) tensors, each in a slot of
    its own; host mirrors of the same arrays for the oracle.  fmt: "f16" or
    "bf16" parameters and gradients; log2_scale: gradients drawn 2^k times
    larger, for the step that unscales them."""

    def __init__(self, torch, cases, v_shift, seed, fmt="f16", log2_scale=None, p_shift=0,
                 g_shift=0):
        self.starts, at = [], 0
        for o, n in cases:
            self.starts.append(at + o)
            at += (o + n + max(v_shift, p_shift, g_shift) + 255) // 256 * 256 + 256
        rng = np.random.default_rng(seed)
        self.cases, self.v_shift, self.fmt, self.k = cases, v_shift, fmt, log2_scale
        self.p_shift, self.g_shift = p_shift, g_shift
        g = rng.standard_normal(at) * 1e-3 * 2.0 ** (log2_scale or 0)
        self.g = (g.astype(np.float16).view(np.uint16) if fmt == "f16"
                  else oracle.f32_to_bf16(g.astype(np.float32)))
        self.w = (rng.standard_normal(at) * 0.02).astype(np.float32)
        self.m = (rng.standard_normal(at) * 1e-4).astype(np.float32)
        self.v = (rng.random(at) * 1e-6).astype(np.float32)
        self.p = np.zeros(at, np.uint16)
        half = torch.float16 if fmt == "f16" else torch.bfloat16
        self.dp = _aligned(torch, at, half)
        self.dg = _aligned(torch, at, half)
        self.dw, self.dm, self.dv = (_aligned(torch, at, torch.float32) for _ in range(3))
        self.dg.copy_(to_dev16(self.g).view(half))
        self.dw.copy_(to_dev32(self.w))
        self.dm.copy_(to_dev32(self.m))
        self.dv.copy_(to_dev32(self.v))

    def tensors(self):
        vs, ps, gs = self.v_shift, self.p_shift, self.g_shift
        return [(self.dp[s + ps:s + ps + n], self.dg[s + gs:s + gs + n], self.dw[s:s + n],
                 self.dm[s:s + n], self.dv[s + vs:s + vs + n])
                for s, (_, n) in zip(self.starts, self.cases)]

    def oracle_step(self, t):
        vs, ps, gs = self.v_shift, self.p_shift, self.g_shift
        for s, (_, n) in zip(self.starts, self.cases):
            p, w, m = self.p[s + ps:s + ps + n], self.w[s:s + n], self.m[s:s + n]
            v, g = self.v[s + vs:s + vs + n], self.g[s + gs:s + gs + n]
            if self.k is None:
                flag = oracle.adam_step(g, p, w, m, v, t=t, fmt=self.fmt, **HP)
            else:
                flag = oracle.adam_step_scaled(g, p, w, m, v, t=t, log2_scale=self.k,
                                               fmt=self.fmt, **HP)
            assert flag == 0

    def compare(self, what):
        """Not-bit-exact elements over every tensor; the parameter buffer
        outside the views (never written) must still be all zero."""
        vs, ps = self.v_shift, self.p_shift
        bad = 0
        gp, gw, gm, gv = host16(self.dp), host32(self.dw), host32(self.dm), host32(self.dv)
        outside = np.ones(gp.size, bool)
        for s, (_, n) in zip(self.starts, self.cases):
            outside[s + ps:s + ps + n] = False
        assert not gp[outside].any(), f"{what}: parameter bytes written outside the views"
        for k, (s, (o, n)) in enumerate(zip(self.starts, self.cases)):
            tag = f"{what} tensor {k} o={o} n={n}"
            r = [check16(gp[s + ps:s + ps + n], self.p[s + ps:s + ps + n], tag + " param",
                         fmt=self.fmt),
                 check32(gw[s:s + n], self.w[s:s + n], tag + " master"),
                 check32(gm[s:s + n], self.m[s:s + n], tag + " m"),
                 check32(gv[s + vs:s + vs + n], self.v[s + vs:s + vs + n], tag + " v")]
            bad += sum(x["not_bit_exact"] for x in r)
        return bad


def _cases(fine):
    """(offset, n) of every tensor.  fine: one aligned tensor of 8M
    elements first and fewer sizes per offset, so that the plan keeps the
    16,384-element chunk (few idle slots) and takes the 256-element tile."""
    if not fine:
        return [(o, n) for o in OFFSETS for n in _sizes(_head(o, 0))]
    few = lambda h: sorted({x for x in (h - 1, h, h + 1, h + 257, h + 16389) if x > 0})
    return [(0, 8 << 20)] + [(o, n) for o in OFFSETS for n in few(_head(o, 0))]


def _want_chunks(cases, v_shift, C):
    return sum(1 + -(-(n - min(n, _head(o, v_shift, n) + C)) // C) for o, n in cases)


@pytest.mark.parametrize("chunk", [0, 512, "fine"])
@pytest.mark.parametrize("v_shift", [0, 4])
def test_heads_match_oracle(zs, chunk, v_shift):
    """A plan over every offset and size; the plan's chunk count shows the
    head it took; two steps, every element of every tensor compared.
    "fine": after one aligned tensor of 8M elements, so the plan keeps the
    16,384-element chunk and the 256-element tile."""
    import torch
    fine = chunk == "fine"
    cases = _cases(fine)
    say(f"tile phase: plan chunk={chunk} v_shift={v_shift} tensors={len(cases)}")
    c = Carved(torch, cases, v_shift, seed=90 + v_shift + (7 if fine else 0))
    plan = zs.zero_plan_create(c.tensors(), 0 if fine else chunk)
    st = plan.stats()
    if fine:
        assert st["tile_elems"] == 256 and st["chunk_elems"] == 16384
    assert st["n_chunks"] == _want_chunks(cases, v_shift, st["chunk_elems"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = 0
    for t in (3, 4):
        zs.zero_adam_step(plan, zs.AdamHParams(**HP), t, flag)
        c.oracle_step(t)
        torch.cuda.synchronize()
        bad += c.compare(f"plan chunk={chunk} v_shift={v_shift} t={t}")
    assert int(flag.item()) == 0
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"
    plan.destroy()


@pytest.mark.parametrize("kind", ["bf16", "f16_scaled", "bf16_scaled"])
def test_heads_other_formats(zs, kind):
    """bfloat16 parameters and gradients, and gradients that carry a loss
    scale of 2^12 (the step multiplies each by 2^-12 first): the same
    kernel template behind the same heads; the library's chunk, two steps,
    every element."""
    import torch
    fmt = "bf16" if kind.startswith("bf16") else "f16"
    k = 12 if kind.endswith("scaled") else None
    cases = _cases(False)
    say(f"tile phase: {kind} tensors={len(cases)}")
    c = Carved(torch, cases, 0, seed=110 + len(kind), fmt=fmt, log2_scale=k)
    plan = zs.zero_plan_create(c.tensors())
    assert plan.stats()["n_chunks"] == _want_chunks(cases, 0, plan.stats()["chunk_elems"])
    ls = zs.LossScale(log2_scale=k, device=torch.device("cuda", 0)) if k is not None else None
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = 0
    for t in (3, 4):
        zs.zero_adam_step(plan, zs.AdamHParams(**HP), t, flag, loss_scale=ls)
        c.oracle_step(t)
        torch.cuda.synchronize()
        bad += c.compare(f"{kind} t={t}")
    assert int(flag.item()) == 0
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"
    plan.destroy()


@pytest.mark.parametrize("v_shift", [0, 4])
def test_heads_noalloc_match_oracle(zs, v_shift):
    """The same tensors through the entry point that builds its chunk table
    in the library's fixed array; two steps, every element."""
    import torch
    cases = _cases(False)
    say(f"tile phase: noalloc v_shift={v_shift} tensors={len(cases)}")
    c = Carved(torch, cases, v_shift, seed=95 + v_shift)
    bad = 0
    for t in (3, 4):
        zs.zero_adam_step_noalloc(c.tensors(), zs.AdamHParams(**HP), t)
        c.oracle_step(t)
        torch.cuda.synchronize()
        bad += c.compare(f"noalloc v_shift={v_shift} t={t}")
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"


@pytest.mark.parametrize("o", [0, 3, 131, 255])
def test_heads_of_the_split_route(zs, o):
    """zero_reduce_adam_step at 32 slices (the reduce, then the one-tensor
    Adam kernel, whose first tile carries the head) with the slices, the
    parameter and the state all o elements into 1 KiB-aligned buffers."""
    import torch
    nd = 32
    h = _head(o, 0)
    rng = np.random.default_rng(400 + o)
    bad = 0
    for n in sorted({1, 5, max(1, h - 1), max(1, h), h + 1, h + 256, h + 257, h + 1024,
                     h + 1025, 70001}):
        say(f"tile phase: split route o={o} n={n} nd={nd}")
        hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
              for _ in range(nd)]
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v0 = (rng.random(n) * 1e-6).astype(np.float32)
        ds = []
        for r in range(nd):
            b = _aligned(torch, n + o, torch.float16)[o:]
            b.copy_(to_dev16(hs[r]))
            ds.append(b)
        p = _aligned(torch, n + o, torch.float16)[o:]
        w, m, v = (_aligned(torch, n + o, torch.float32)[o:] for _ in range(3))
        w.copy_(to_dev32(w0))
        m.copy_(to_dev32(m0))
        v.copy_(to_dev32(v0))
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        zs.zero_reduce_adam_step(ds, p, w, m, v, zs.AdamHParams(**HP), 3, nonfinite_flag=flag)
        g_ref, rflag = oracle.reduce_grad(hs)
        p_ref = np.zeros(n, np.uint16)
        aflag = oracle.adam_step(g_ref, p_ref, w0, m0, v0, t=3, **HP)
        torch.cuda.synchronize()
        what = f"split o={o} n={n}"
        r = [check16(host16(p), p_ref, what + " param"), check32(host32(w), w0, what + " master"),
             check32(host32(m), m0, what + " m"), check32(host32(v), v0, what + " v")]
        bad += sum(x["not_bit_exact"] for x in r)
        assert int(flag.item()) == (rflag | aflag)
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"
