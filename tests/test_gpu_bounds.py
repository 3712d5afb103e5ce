"""Every GPU entry point writes exactly its outputs: nothing outside them and
every element of them.

Element-by-element parity against the oracle cannot see a kernel that
writes past the end of an array into memory the test does not compare.
Here every array of a call is carved out of one device buffer with guard
zones before and after it, all filled with a byte pattern; after the call
the guards must still hold it.  Write-only outputs (fp16 parameters,
reduced gradients, the gathered buffer) are pre-filled with a NaN pattern
no finite input produces, and afterwards none of it may remain.  The
arrays cover every access path (phases in a 16-byte vector, one element
off) and ragged sizes around the tiles (1 to 70,001 elements), for fp16
and bfloat16.  Each case prints its name before it touches the GPU."""
import numpy as np
import pytest

from zero_partitioned_mixed_layout_amd import workloads as W

pytestmark = pytest.mark.gpu
HP = dict(W.ADAM_HP)
GUARD = 4096          # guard bytes before and after every array
FILL = 0xA5           # guard byte pattern
UNWRITTEN = 0x7E01    # a NaN payload no finite input produces (fp16 and bfloat16 NaN alike)
SIZES = (1, 3, 5, 255, 256, 257, 511, 513, 4099, 16391, 70001)


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


class Arena:
    """Arrays carved out of one byte buffer, each with a guard zone before
    and after it; `phase` shifts an array's start by that many bytes from a
    multiple of `unit` bytes (256 or 1024) past the buffer's first 1 KiB
    boundary."""

    def __init__(self, specs, unit=256):
        import torch
        self.spans, off = [], GUARD
        for nbytes, phase in specs:
            self.spans.append((off + phase, nbytes))
            off += (phase + nbytes + unit - 1) // unit * unit + GUARD
        self.raw = torch.full((off + 1024,), FILL, dtype=torch.uint8, device="cuda")
        base = (-self.raw.data_ptr()) % 1024
        self.spans = [(lo + base, nbytes) for lo, nbytes in self.spans]

    def view(self, k, dtype):
        lo, nbytes = self.spans[k]
        return self.raw[lo:lo + nbytes].view(dtype)

    def check(self, what):
        h = self.raw.cpu().numpy()
        mask = np.ones(h.size, bool)
        for lo, nbytes in self.spans:
            mask[lo:lo + nbytes] = False
        bad = np.flatnonzero(mask & (h != FILL))
        assert bad.size == 0, f"{what}: {bad.size} guard bytes written, first at {bad[:8]}"


def _half(fmt):
    import torch
    return torch.float16 if fmt == "f16" else torch.bfloat16


def _randn16(torch, t, seed, std=1e-3):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t.copy_(torch.randn(t.numel(), generator=g, device="cuda") * std)


def _all_written(t, what):
    import torch
    left = int((t.view(torch.int16) == np.int16(UNWRITTEN)).sum().item())
    assert left == 0, f"{what}: {left} elements never written"


# byte phases of (param, grad, master, m, v): vector path, a peeled head,
# and the parameter one element off the state (single path); "kib_head":
# every array 131 elements into a 1 KiB slot, so the fp32 arrays reach
# their next 1 KiB boundary together and the head runs 125 elements (one
# singly, then 31 groups of four)
ADAM_LAYOUTS = {"aligned": (0, 0, 0, 0, 0), "head": (6, 6, 12, 12, 12),
                "param_off": (2, 0, 0, 0, 0), "kib_head": (262, 262, 524, 524, 524)}
UNITS = {"kib_head": 1024}


def _adam_arena(torch, sizes, layout, fmt, seed):
    po, go, wo, mo, vo = ADAM_LAYOUTS[layout]
    specs = []
    for n in sizes:
        specs += [(2 * n, po), (2 * n, go), (4 * n, wo), (4 * n, mo), (4 * n, vo)]
    A = Arena(specs, UNITS.get(layout, 256))
    tensors = []
    for k, n in enumerate(sizes):
        p, g = A.view(5 * k, _half(fmt)), A.view(5 * k + 1, _half(fmt))
        w, m, v = (A.view(5 * k + j, torch.float32) for j in (2, 3, 4))
        p.view(torch.int16).fill_(UNWRITTEN)
        _randn16(torch, g, seed + k)
        _randn16(torch, w, seed + 100 + k, 0.02)
        m.zero_()
        v.zero_()
        tensors.append((p, g, w, m, v))
    return A, tensors


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", list(ADAM_LAYOUTS))
@pytest.mark.parametrize("chunk", [0, 512])
def test_adam_plan_bounds(zs, fmt, layout, chunk):
    """zero_adam_step over a plan of every ragged size at once (the
    library's chunk choice, and 512-element chunks with their coarse tile),
    then the scaled step over the same plan."""
    import torch
    say(f"bounds: Adam plan fmt={fmt} layout={layout} chunk={chunk}")
    A, tensors = _adam_arena(torch, SIZES, layout, fmt, 11)
    plan = zs.zero_plan_create(tensors, chunk)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1, flag)
    torch.cuda.synchronize()
    A.check(f"Adam {fmt} {layout} chunk {chunk}")
    for k, t in enumerate(tensors):
        _all_written(t[0], f"Adam {fmt} {layout} tensor {k} param")
    ls = zs.LossScale(log2_scale=3, device=torch.device("cuda", 0))
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 2, flag, loss_scale=ls)
    torch.cuda.synchronize()
    A.check(f"scaled Adam {fmt} {layout} chunk {chunk}")
    plan.destroy()


@pytest.mark.parametrize("layout", ["aligned", "head", "kib_head"])
def test_adam_plan_bounds_fine_tile(zs, layout):
    """Big vector tensors (the library's 16,384-element chunk), which take
    the 256-element Adam tile."""
    import torch
    say(f"bounds: Adam plan, fine tile, layout={layout}")
    A, tensors = _adam_arena(torch, (1_000_003, 2_000_001), layout, "f16", 13)
    plan = zs.zero_plan_create(tensors)
    assert plan.stats()["tile_elems"] == 256
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1)
    torch.cuda.synchronize()
    A.check(f"Adam fine tile {layout}")
    for k, t in enumerate(tensors):
        _all_written(t[0], f"Adam fine tile {layout} tensor {k} param")
    plan.destroy()


@pytest.mark.parametrize("layout", list(ADAM_LAYOUTS))
def test_adam_noalloc_bounds(zs, layout):
    """zero_adam_step_noalloc over every ragged size, twice (the second call
    over fewer tensors)."""
    import torch
    say(f"bounds: Adam noalloc layout={layout}")
    A, tensors = _adam_arena(torch, SIZES, layout, "f16", 12)
    zs.zero_adam_step_noalloc(tensors, zs.AdamHParams(**HP), 1)
    torch.cuda.synchronize()
    A.check(f"noalloc {layout}")
    for k, t in enumerate(tensors):
        _all_written(t[0], f"noalloc {layout} tensor {k} param")
    zs.zero_adam_step_noalloc(tensors[::3], zs.AdamHParams(**HP), 2)
    torch.cuda.synchronize()
    A.check(f"noalloc {layout}, second call")


# byte phases of (even slices, odd slices, output): 16-byte, 8-byte (every
# other slice or every slice 8 bytes off the output's 16-byte phase) and
# 2-byte common phases (the reduce's three paths)
REDUCE_LAYOUTS = {"v16": (0, 0, 0), "v8": (0, 8, 0), "v8_all": (8, 8, 0), "single": (0, 0, 2)}


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", list(REDUCE_LAYOUTS))
@pytest.mark.parametrize("nd", [1, 2, 3, 4, 7, 15, 17, 19, 64])
def test_reduce_bounds(zs, fmt, layout, nd):
    import torch
    say(f"bounds: reduce fmt={fmt} layout={layout} nd={nd}")
    se, so, oo = REDUCE_LAYOUTS[layout]
    for n in SIZES:
        A = Arena([(2 * n, se if r % 2 == 0 else so) for r in range(nd)] + [(2 * n, oo)])
        sl = [A.view(r, _half(fmt)) for r in range(nd)]
        for r, s in enumerate(sl):
            _randn16(torch, s, 300 + r)
        out = A.view(nd, _half(fmt))
        out.view(torch.int16).fill_(UNWRITTEN)
        zs.zero_reduce_grad_shard(sl, out)
        torch.cuda.synchronize()
        A.check(f"reduce {fmt} {layout} nd={nd} n={n}")
        _all_written(out, f"reduce {fmt} {layout} nd={nd} n={n}")


# byte phases of (even slices, odd slices, param, grad_out, master, m, v);
# "kib_head" in 1 KiB slots, as for the Adam step
FUSED_LAYOUTS = {"aligned": (0, 0, 0, 0, 0, 0, 0), "phase": (4, 4, 4, 4, 8, 8, 8),
                 "split": (0, 8, 0, 0, 0, 0, 0), "odd": (2, 2, 0, 0, 0, 0, 0),
                 "param_off": (0, 0, 2, 2, 0, 0, 0),
                 "kib_head": (262, 262, 262, 262, 524, 524, 524)}


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", list(FUSED_LAYOUTS))
@pytest.mark.parametrize("nd", [4, 8, 16, 31, 32, 64])
def test_fused_bounds(zs, fmt, layout, nd):
    """zero_reduce_adam_step on both sides of its split (one fused kernel
    below ZERO_FUSED_SPLIT_SLICES slices, the reduce and the one-tensor Adam
    kernel from there on), with and without the gradient output."""
    import torch
    say(f"bounds: fused fmt={fmt} layout={layout} nd={nd}")
    se, so, po, go, wo, mo, vo = FUSED_LAYOUTS[layout]
    for n in SIZES:
        for with_gout in (False, True):
            specs = [(2 * n, se if r % 2 == 0 else so) for r in range(nd)]
            specs += [(2 * n, po), (2 * n, go), (4 * n, wo), (4 * n, mo), (4 * n, vo)]
            A = Arena(specs, UNITS.get(layout, 256))
            sl = [A.view(r, _half(fmt)) for r in range(nd)]
            for r, s in enumerate(sl):
                _randn16(torch, s, 500 + r)
            p, gout = A.view(nd, _half(fmt)), A.view(nd + 1, _half(fmt))
            w, m, v = (A.view(nd + j, torch.float32) for j in (2, 3, 4))
            p.view(torch.int16).fill_(UNWRITTEN)
            gout.view(torch.int16).fill_(UNWRITTEN)
            _randn16(torch, w, 600, 0.02)
            m.zero_()
            v.zero_()
            zs.zero_reduce_adam_step(sl, p, w, m, v, zs.AdamHParams(**HP), 1,
                                     grad_out=gout if with_gout else None)
            torch.cuda.synchronize()
            what = f"fused {fmt} {layout} nd={nd} n={n} gout={with_gout}"
            A.check(what)
            _all_written(p, what + " param")
            if with_gout:
                _all_written(gout, what + " grad_out")


@pytest.mark.parametrize("layout", ["aligned", "dst_off", "src_off"])
def test_gather_bounds(zs, layout):
    """zero_gather_shards into a full buffer (destination on a line, or one
    element off it; sources at other phases, read shifted from 1,024
    elements, whole aligned words that may reach past a shard's ends), every
    shard moved except the one already in place."""
    import torch
    say(f"bounds: gather layout={layout}")
    for S in (1, 63, 64, 65, 1026, 2047, 2048, 2049, 4099, 5000):
        nd = 5
        fo = 2 if layout == "dst_off" else 0
        specs = [(2 * S * nd, fo)] + [(2 * S, 2 * (r % 3) if layout == "src_off" else 0)
                                      for r in range(nd)]
        A = Arena(specs)
        full = A.view(0, torch.float16)
        full.view(torch.int16).fill_(UNWRITTEN)
        shards = [A.view(1 + r, torch.float16) for r in range(nd)]
        for r, s in enumerate(shards):
            _randn16(torch, s, 700 + r)
        # rank 2's shard is already in place
        full[2 * S:3 * S].copy_(shards[2])
        shards[2] = full[2 * S:3 * S]
        zs.zero_gather_shards(shards, full)
        torch.cuda.synchronize()
        A.check(f"gather {layout} S={S}")
        _all_written(full, f"gather {layout} S={S}")


def test_loss_scale_update_bounds(zs):
    """zero_loss_scale_update writes the 16-byte record and the flag only."""
    import torch
    say("bounds: loss-scale update")
    A = Arena([(16, 0), (4, 0)])
    rec = A.view(0, torch.int32)
    flag = A.view(1, torch.int32)
    rec.copy_(torch.tensor([16, 0, 0, 0], dtype=torch.int32))
    for f in (1, 0, 0):
        flag.fill_(f)
        lib = zs.lib()
        rc = lib.zero_loss_scale_update(rec.data_ptr(), flag.data_ptr(), 2, -4, 24,
                                        torch.cuda.current_stream().cuda_stream)
        assert rc == 0
    torch.cuda.synchronize()
    A.check("loss-scale update")
    assert rec.cpu().tolist() == [16, 0, 1, 2] and int(flag.item()) == 0
