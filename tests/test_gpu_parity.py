"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
small and ragged inputs: every element compared.  Each case prints its name
and sizes before it touches the GPU."""
import numpy as np
import pytest

import oracle
from parity import check16, check32, host16, host32, to_dev16, to_dev32
from zero_partitioned_mixed_layout_amd import workloads as W

pytestmark = pytest.mark.gpu

HP = dict(W.ADAM_HP)


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


@pytest.fixture(scope="module")
def torch_mod(zs):
    import torch
    return torch


def _hp(zs):
    return zs.AdamHParams(**HP)


class HostShard:
    """Host copies of one tensor's five arrays for the oracle."""

    def __init__(self, g16, p16, w, m, v):
        self.g, self.p, self.w, self.m, self.v = g16, p16, w, m, v

    def step(self, t, skip=False):
        return oracle.adam_step(self.g, self.p, self.w, self.m, self.v, t=t, skip=skip, **HP)


def _compare(dev_arrays, host: HostShard, what):
    p, g, w, m, v = dev_arrays
    r = [check16(host16(p), host.p, f"{what} param"), check32(host32(w), host.w, f"{what} master"),
         check32(host32(m), host.m, f"{what} m"), check32(host32(v), host.v, f"{what} v")]
    return sum(x["not_bit_exact"] for x in r)


def test_tiny_flat_ten_steps(zs, torch_mod):
    """2^20 parameters over 4 ranks: rank 0's 262,144-element shard, 10 steps,
    all elements compared after every step (underflow and swamping sets
    included)."""
    torch = torch_mod
    wl = W.WORKLOADS["tiny_flat"]
    lay = zs.zero_shard_layout(wl.psi, wl.nd, wl.rank, wl.align)
    assert lay._asdict() == oracle.shard_layout(wl.psi, wl.nd, wl.rank, wl.align)
    n = lay.real_len
    say(f"tiny_flat n={n} steps={wl.steps}")
    master, m, v, p16 = W.tiny_initial_state(wl)
    host = HostShard(None, p16.view(np.uint16).copy(), master.copy(), m.copy(), v.copy())
    full = torch.zeros(lay.padded_total, dtype=torch.float16, device="cuda")
    dp = full[lay.offset:lay.offset + n]
    dp.copy_(to_dev16(p16.view(np.uint16)))
    dg = torch.empty(n, dtype=torch.float16, device="cuda")
    dw, dm, dv = to_dev32(master), to_dev32(m), to_dev32(v)
    plan = zs.zero_plan_create([(dp, dg, dw, dm, dv)])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    inexact = 0
    for t in range(1, wl.steps + 1):
        g = W.tiny_grad16(wl, t)
        dg.copy_(to_dev16(g.view(np.uint16)))
        zs.zero_adam_step(plan, _hp(zs), t, flag)
        host.g = g.view(np.uint16)
        assert host.step(t) == 0
        torch.cuda.synchronize()
        inexact += _compare((dp, dg, dw, dm, dv), host, f"tiny t={t}")
    assert int(flag.item()) == 0
    # the rest of the full fp16 buffer (other ranks' shards) is untouched
    assert int(torch.count_nonzero(full[n:]).item()) == 0
    assert inexact == 0, f"{inexact} elements within tolerance but not bit-exact"
    plan.destroy()


def _ragged_plan(zs, torch, sizes_offsets, seed, warm=False):
    """Tensors of the given sizes, each array a view at its own element
    offset into a larger buffer (so the five arrays of a tensor can disagree
    in alignment).  Returns device arrays, host mirrors."""
    rng = np.random.default_rng(seed)
    dev, host = [], []
    for k, (n, offs) in enumerate(sizes_offsets):
        bufs = []
        for j, (o, dt) in enumerate(zip(offs, (torch.float16, torch.float16, torch.float32,
                                               torch.float32, torch.float32))):
            bufs.append(torch.zeros(n + o + 8, dtype=dt, device="cuda")[o:o + n])
        p, g, w, m, v = bufs
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32) if warm else np.zeros(n, np.float32)
        v0 = (rng.random(n) * 1e-6).astype(np.float32) if warm else np.zeros(n, np.float32)
        w.copy_(to_dev32(w0))
        m.copy_(to_dev32(m0))
        v.copy_(to_dev32(v0))
        dev.append((p, g, w, m, v))
        host.append(HostShard(None, np.zeros(n, np.uint16), w0.copy(), m0.copy(), v0.copy()))
    return dev, host


SIZES = [1, 7, 8, 9, 31, 255, 256, 257, 511, 512, 513, 4095, 4096, 4097, 2048 * 3 + 5, 70001, 0]
# element offsets of (param, grad, master, m, v) inside their buffers
OFFSETS = [(0, 0, 0, 0, 0),      # all aligned: vector path, no head
           (4, 0, 0, 0, 0),      # param 8 mod 16 bytes, grad 0: vector path, no head
           (3, 3, 3, 3, 3),      # common phase: peel 1, then vectors
           (2, 6, 2, 2, 6),      # phases agree mod a vector: peel 2, then vectors
           (1, 0, 0, 0, 0),      # param one element off: single elements
           (0, 0, 1, 0, 0)]      # master 4 mod 16 bytes: single elements


@pytest.mark.parametrize("chunk", [0, 512, 1536, "fine"])
@pytest.mark.parametrize("warm", [False, True])
def test_ragged_sizes_and_alignments(zs, torch_mod, warm, chunk):
    """One plan over tensors of sizes 0..70001 whose arrays sit at every
    alignment class, with the default chunk size and with chunks of 512 and
    1536 elements (one and three tiles: many chunk boundaries inside small
    tensors), all on 512-element tiles; "fine": the same tensors after one
    aligned tensor of 8M elements, which keeps the plan's chunk at 16384
    and its tile at 256 elements.  Sizes on both sides of both tiles;
    three steps; every element compared."""
    torch = torch_mod
    so = [(n, OFFSETS[i % len(OFFSETS)]) for i, n in enumerate(SIZES)]
    so += [(n, OFFSETS[(i + 2) % len(OFFSETS)]) for i, n in enumerate(SIZES)]
    fine = chunk == "fine"
    if fine:
        so = [(8 << 20, OFFSETS[0])] + so
        chunk = 0
    say(f"ragged warm={warm} chunk={chunk} fine={fine} tensors={len(so)}")
    dev, host = _ragged_plan(zs, torch, so, seed=42 + warm, warm=warm)
    plan = zs.zero_plan_create(dev, chunk)
    st = plan.stats()
    assert st["tile_elems"] == (256 if fine else 512)
    assert (st["chunk_elems"] == 16384) if fine else True
    assert st["vector_elems"] and st["scalar_elems"]
    assert st["vector_elems"] + st["scalar_elems"] == st["n_params"]
    rng = np.random.default_rng(7)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    t0 = 6 if warm else 1
    inexact = 0
    for t in range(t0, t0 + 3):
        for (p, g, w, m, v), h in zip(dev, host):
            gh = (rng.standard_normal(w.numel()) * 1e-3).astype(np.float16).view(np.uint16)
            if w.numel():
                g.copy_(to_dev16(gh))
            h.g = gh
        zs.zero_adam_step(plan, _hp(zs), t, flag)
        for h in host:
            h.step(t)
        torch.cuda.synchronize()
        for k, (d, h) in enumerate(zip(dev, host)):
            if d[2].numel():
                inexact += _compare(d, h, f"ragged tensor {k} n={d[2].numel()} t={t}")
    assert int(flag.item()) == 0
    assert inexact == 0
    plan.destroy()


def test_every_fp16_gradient_pattern(zs, torch_mod):
    """All 65,536 fp16 bit patterns as gradients (subnormals, +-0, +-inf,
    NaNs) in one step from a warm state; non-finite ones must give the
    oracle's IEEE classes and raise the flag."""
    torch = torch_mod
    n = 1 << 16
    say("every fp16 gradient pattern")
    rng = np.random.default_rng(5)
    g = np.arange(n, dtype=np.uint32).astype(np.uint16)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-6).astype(np.float32)
    host = HostShard(g, np.zeros(n, np.uint16), w0.copy(), m0.copy(), v0.copy())
    dp = torch.zeros(n, dtype=torch.float16, device="cuda")
    dg, dw, dm, dv = to_dev16(g), to_dev32(w0), to_dev32(m0), to_dev32(v0)
    plan = zs.zero_plan_create([(dp, dg, dw, dm, dv)])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, _hp(zs), 3, flag)
    assert host.step(3) == 1
    torch.cuda.synchronize()
    assert _compare((dp, dg, dw, dm, dv), host, "all patterns") == 0
    assert int(flag.item()) == 1
    plan.destroy()


@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00, 0xFD55])
@pytest.mark.parametrize("where", ["head", "body", "tail"])
def test_flag_per_class_and_position(zs, torch_mod, bad, where):
    """One non-finite gradient, in a peeled head element, a vector body or
    a ragged tail, raises the flag; finite gradients leave it at 0."""
    torch = torch_mod
    n = 4096 + 3
    say(f"flag bad={bad:#x} where={where}")
    buf16 = [torch.zeros(n + 8, dtype=torch.float16, device="cuda")[3:3 + n] for _ in range(2)]
    buf32 = [torch.zeros(n + 8, dtype=torch.float32, device="cuda")[3:3 + n] for _ in range(3)]
    g = np.full(n, 0x1400, np.uint16)
    pos = {"head": 1, "body": 2000, "tail": n - 1}[where]
    buf16[1].copy_(to_dev16(g))
    plan = zs.zero_plan_create([(buf16[0], buf16[1], *buf32)])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, _hp(zs), 1, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    g[pos] = bad
    buf16[1].copy_(to_dev16(g))
    zs.zero_adam_step(plan, _hp(zs), 2, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    plan.destroy()


def test_skip_writes_nothing(zs, torch_mod):
    torch = torch_mod
    n = 10000
    say("skip")
    rng = np.random.default_rng(9)
    arrays = [to_dev16(rng.integers(0, 0x7000, n, dtype=np.uint16)),
              to_dev16((rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)),
              to_dev32(rng.standard_normal(n)), to_dev32(rng.standard_normal(n)),
              to_dev32(rng.random(n))]
    before = [a.clone() for a in arrays]
    plan = zs.zero_plan_create([arrays])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    skip = torch.ones(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, _hp(zs), 4, flag, skip)
    torch.cuda.synchronize()
    for a, b in zip(arrays, before):
        assert torch.equal(a.view(torch.int16 if a.dtype == torch.float16 else torch.int32),
                           b.view(torch.int16 if b.dtype == torch.float16 else torch.int32))
    assert int(flag.item()) == 0
    skip.zero_()
    zs.zero_adam_step(plan, _hp(zs), 4, flag, skip)
    torch.cuda.synchronize()
    assert not torch.equal(arrays[2], before[2])
    with pytest.raises(zs.ZeroError):
        zs.zero_adam_step(plan, _hp(zs), 4, flag, flag)       # flag == skip
    plan.destroy()


def test_resume_is_bit_exact(zs, torch_mod):
    """10 steps == 5 steps, a copy of all five arrays into fresh tensors, a
    new plan, and 5 more steps continuing t."""
    torch = torch_mod
    n = 50000
    say("resume 5+5")
    rng = np.random.default_rng(11)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [to_dev16((rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16))
             for _ in range(10)]

    def fresh():
        return [torch.zeros(n, dtype=torch.float16, device="cuda"),
                torch.zeros(n, dtype=torch.float16, device="cuda"),
                to_dev32(w0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")]

    a = fresh()
    pa = zs.zero_plan_create([a])
    for t in range(1, 11):
        a[1].copy_(grads[t - 1])
        zs.zero_adam_step(pa, _hp(zs), t, None)
    b = fresh()
    pb = zs.zero_plan_create([b])
    for t in range(1, 6):
        b[1].copy_(grads[t - 1])
        zs.zero_adam_step(pb, _hp(zs), t, None)
    c = [x.clone() for x in b]
    pc = zs.zero_plan_create([c])
    for t in range(6, 11):
        c[1].copy_(grads[t - 1])
        zs.zero_adam_step(pc, _hp(zs), t, None)
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert torch.equal(x.view(torch.int16 if x.dtype == torch.float16 else torch.int32),
                           y.view(torch.int16 if y.dtype == torch.float16 else torch.int32))
    for p in (pa, pb, pc):
        p.destroy()


# --------------------------------------------------------------------------
# Gradient reduction.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("nd", [1, 2, 3, 4, 5, 8, 9, 16, 17, 64, 256])
@pytest.mark.parametrize("layout", ["aligned", "phase3", "mixed4", "mixed4h", "odd"])
def test_reduce_matches_oracle(zs, torch_mod, nd, layout):
    """Every output element of the N_d-slice average, for N_d from 1 to
    256, sizes with ragged tails (1027 = a head of 3 and two whole 512-element
    tiles under "mixed4h"), and slice alignments that select each access
    path (16-byte, peeled head, 8-byte with and without a head, single
    element)."""
    torch = torch_mod
    rng = np.random.default_rng(1000 + nd)
    for n in (1, 7, 9, 1027, 4097, 65537):
        say(f"reduce nd={nd} layout={layout} n={n}")
        hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16) for _ in range(nd)]
        offs = {"aligned": [0] * (nd + 1), "phase3": [3] * (nd + 1),
                "mixed4": [4 * (r % 2) for r in range(nd + 1)],
                "mixed4h": [1 + 4 * (r % 2) for r in range(nd + 1)],
                "odd": [r % 3 for r in range(nd + 1)]}[layout]
        ds = []
        for r in range(nd):
            b = torch.zeros(n + 8, dtype=torch.float16, device="cuda")[offs[r]:offs[r] + n]
            b.copy_(to_dev16(hs[r]))
            ds.append(b)
        out = torch.zeros(n + 8, dtype=torch.float16, device="cuda")[offs[nd]:offs[nd] + n]
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        zs.zero_reduce_grad_shard(ds, out, flag)
        ref, rflag = oracle.reduce_grad(hs)
        torch.cuda.synchronize()
        r = check16(host16(out), ref, f"reduce nd={nd} n={n} {layout}")
        assert r["not_bit_exact"] == 0
        assert int(flag.item()) == rflag == 0


@pytest.mark.parametrize("nd", [4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, 18, 23, 31, 47])
@pytest.mark.parametrize("oshift", [0, 3])
@pytest.mark.parametrize("phase", ["aligned", "mixed4", "odd"])
def test_reduce_every_batch_size(zs, torch_mod, nd, oshift, phase):
    """The 16- and 8-byte paths load batches of 16 slices and then the rest
    in one batch, the single-element path batches of 8 and then the rest:
    every rest of 1-15 slices (after zero, one and two batches of 16),
    slices 16-byte aligned, every other one 8 bytes off, or at r mod 3
    elements (no common phase), the output in the slices' phase and three
    elements off it, against the oracle bit for bit; a non-finite value in
    the last slice of the rest raises the flag."""
    torch = torch_mod
    rng = np.random.default_rng(5000 + nd)
    n = 9 * 512 + 13
    say(f"reduce batches nd={nd} oshift={oshift} phase={phase} n={n}")
    hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16) for _ in range(nd)]
    ds = []
    for r, h in enumerate(hs):
        o = 4 * (r % 2) if phase == "mixed4" else (r % 3 if phase == "odd" else 0)
        b = torch.zeros(n + 8, dtype=torch.float16, device="cuda")[o:o + n]
        b.copy_(to_dev16(h))
        ds.append(b)
    obuf = torch.zeros(n + 8, dtype=torch.float16, device="cuda")
    out = obuf[oshift:oshift + n]
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_grad_shard(ds, out, flag)
    ref, rflag = oracle.reduce_grad(hs)
    torch.cuda.synchronize()
    assert check16(host16(out), ref, f"reduce nd={nd}")["not_bit_exact"] == 0
    assert int(flag.item()) == rflag == 0
    assert not host16(obuf[:oshift]).any() and not host16(obuf[oshift + n:]).any()
    hs[-1][n // 2] = 0x7C00
    ds[-1].copy_(to_dev16(hs[-1]))
    zs.zero_reduce_grad_shard(ds, out, flag)
    ref, rflag = oracle.reduce_grad(hs)
    torch.cuda.synchronize()
    assert check16(host16(out), ref, f"reduce nd={nd} inf")["not_bit_exact"] == 0
    assert int(flag.item()) == rflag == 1


def test_reduce_special_values(zs, torch_mod):
    """N_d = 1 copies all 65,536 patterns; +inf with -inf gives NaN and the
    flag; the fp32 sum does not overflow where the fp16 mean fits."""
    torch = torch_mod
    say("reduce special values")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    out = torch.zeros(1 << 16, dtype=torch.float16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_grad_shard([to_dev16(bits)], out, flag)
    ref, rflag = oracle.reduce_grad([bits])
    torch.cuda.synchronize()
    check16(host16(out), ref, "nd=1 copy")
    assert int(flag.item()) == rflag == 1
    a = np.array([0x7C00, 0x7BFF, 0x3C00, 0x0001] * 3, np.uint16)
    b = np.array([0xFC00, 0x7BFF, 0x3C00, 0x8001] * 3, np.uint16)
    out = torch.zeros(a.size, dtype=torch.float16, device="cuda")
    flag.zero_()
    zs.zero_reduce_grad_shard([to_dev16(a), to_dev16(b)], out, flag)
    ref, rflag = oracle.reduce_grad([a, b])
    torch.cuda.synchronize()
    check16(host16(out), ref, "inf mix")
    assert int(flag.item()) == rflag == 1


def test_reduce_then_step_skips_on_nonfinite(zs, torch_mod):
    """The reduce's flag chained as the step's skip input: an infinite
    gradient slice leaves every state array untouched."""
    torch = torch_mod
    say("reduce -> skip chain")
    n = 3000
    rng = np.random.default_rng(3)
    hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16) for _ in range(4)]
    hs[2][1234] = 0x7C00
    ds = [to_dev16(h) for h in hs]
    grad = torch.zeros(n, dtype=torch.float16, device="cuda")
    st = [torch.zeros(n, dtype=torch.float16, device="cuda"), grad,
          to_dev32(rng.standard_normal(n)), to_dev32(rng.standard_normal(n) * 1e-3),
          to_dev32(rng.random(n) * 1e-6)]
    before = [x.clone() for x in st]
    reduce_flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    step_flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = zs.zero_plan_create([st])
    zs.zero_reduce_grad_shard(ds, grad, reduce_flag)
    zs.zero_adam_step(plan, _hp(zs), 2, step_flag, reduce_flag)
    torch.cuda.synchronize()
    assert int(reduce_flag.item()) == 1 and int(step_flag.item()) == 0
    assert torch.equal(st[0].view(torch.int16), before[0].view(torch.int16))
    for k in (2, 3, 4):
        assert torch.equal(st[k].view(torch.int32), before[k].view(torch.int32))
    plan.destroy()


def test_rejects_through_binding(zs, torch_mod):
    torch = torch_mod
    a = torch.zeros(16, dtype=torch.float16, device="cuda")
    with pytest.raises(zs.ZeroError):
        zs.zero_reduce_grad_shard([a[:8], a[8:16]], a[2:10])      # out overlaps a slice
    w = torch.zeros(16, device="cuda")
    with pytest.raises(zs.ZeroError):                          # m aliases master
        zs.zero_plan_create([(a, a.clone(), w, w, torch.zeros(16, device="cuda"))])
    with pytest.raises(TypeError):
        zs.zero_plan_create([(a, a.clone(), w.half(), w.clone(), w.clone())])


def test_two_plans_on_two_streams(zs, torch_mod):
    """The library keeps no mutable state between calls: two ranks' shards,
    each with its own plan, slices and flags, stepped on two streams at once
    (reduce, then Adam with the reduce's flag as skip input, three steps
    each, launches interleaved across the streams) equal the oracle run
    separately on each."""
    torch = torch_mod
    say("two plans on two streams")
    rng = np.random.default_rng(77)
    sizes = (300_001, 123_457)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    nd = 3
    shards, hosts, plans = [], [], []
    for n in sizes:
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        dev = dict(p=torch.zeros(n, dtype=torch.float16, device="cuda"),
                   g=torch.zeros(n, dtype=torch.float16, device="cuda"),
                   w=to_dev32(w0), m=torch.zeros(n, device="cuda"), v=torch.zeros(n, device="cuda"),
                   rflag=torch.zeros(1, dtype=torch.int32, device="cuda"),
                   aflag=torch.zeros(1, dtype=torch.int32, device="cuda"))
        shards.append(dev)
        hosts.append(HostShard(np.zeros(n, np.uint16), np.zeros(n, np.uint16), w0.copy(),
                               np.zeros(n, np.float32), np.zeros(n, np.float32)))
        plans.append(zs.zero_plan_create([(dev["p"], dev["g"], dev["w"], dev["m"], dev["v"])]))
    torch.cuda.synchronize()
    for t in (1, 2, 3):
        slices = []
        for k, n in enumerate(sizes):
            hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16) for _ in range(nd)]
            slices.append((hs, [to_dev16(h) for h in hs]))
        torch.cuda.synchronize()                  # inputs are in place before either stream starts
        for k in (0, 1):                          # the two reduces, one per stream
            with torch.cuda.stream(streams[k]):
                zs.zero_reduce_grad_shard(slices[k][1], shards[k]["g"], shards[k]["rflag"])
        for k in (0, 1):                          # then the two steps, each after its own reduce
            with torch.cuda.stream(streams[k]):
                zs.zero_adam_step(plans[k], _hp(zs), t, shards[k]["aflag"], shards[k]["rflag"])
        for k in (0, 1):
            g_ref, _ = oracle.reduce_grad(slices[k][0])
            hosts[k].g[:] = g_ref
            hosts[k].step(t)
        torch.cuda.synchronize()
    for k in (0, 1):
        d = shards[k]
        assert _compare((d["p"], d["g"], d["w"], d["m"], d["v"]), hosts[k], f"stream {k}") == 0
        assert int(d["rflag"].item()) == 0 and int(d["aflag"].item()) == 0
        plans[k].destroy()


def test_fp32_subnormal_state_is_kept(zs, torch_mod):
    """Master, m and v at fp32 subnormals and just above the smallest normal,
    gradients 0, +-2^-24 (the smallest fp16 subnormal) or small normals, at
    t = 7: the kernel keeps subnormals (built without flushing them to
    zero), bit for bit with the oracle.  The oracle's results must contain
    subnormal m and v, so the case is exercised."""
    torch = torch_mod
    say("fp32 subnormal state")
    n = 70_001
    rng = np.random.default_rng(38)

    def tiny(k):
        # subnormal bit patterns and the first normals, either sign
        b = rng.integers(1, 0x01000000, size=k, dtype=np.uint64).astype(np.uint32)
        b |= (rng.random(k) < 0.5).astype(np.uint32) << 31
        return b.view(np.float32)

    w0, m0 = tiny(n), tiny(n)
    v0 = np.abs(tiny(n))
    choice = rng.integers(0, 4, n)
    g = np.where(choice == 0, 0, np.where(choice == 1, 0x0001, np.where(choice == 2, 0x8001, 0x0400))).astype(np.uint16)
    host = HostShard(g.copy(), np.zeros(n, np.uint16), w0.copy(), m0.copy(), v0.copy())
    flag_ref = host.step(7)
    m_sub = (host.m != 0) & (np.abs(host.m) < np.finfo(np.float32).tiny)
    v_sub = (host.v != 0) & (host.v < np.finfo(np.float32).tiny)
    assert m_sub.sum() > 1000 and v_sub.sum() > 1000
    p = torch.zeros(n, dtype=torch.float16, device="cuda")
    dev = (p, to_dev16(g), to_dev32(w0), to_dev32(m0), to_dev32(v0))
    plan = zs.zero_plan_create([dev])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, _hp(zs), 7, flag)
    torch.cuda.synchronize()
    assert _compare(dev, host, "subnormal state") == 0
    assert int(flag.item()) == flag_ref == 0
    plan.destroy()
    # the reduce keeps fp16 subnormal slices exact too (sums of a few 2^-24)
    hs = [rng.choice(np.array([0x0000, 0x0001, 0x8001, 0x0002, 0x03FF], np.uint16), size=n) for _ in range(3)]
    out = torch.zeros(n, dtype=torch.float16, device="cuda")
    rflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_grad_shard([to_dev16(h) for h in hs], out, rflag)
    ref, _ = oracle.reduce_grad(hs)
    torch.cuda.synchronize()
    assert np.array_equal(host16(out), ref)


@pytest.mark.parametrize("hp", [
    dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8),
    dict(lr=0.1, beta1=0.0, beta2=0.0, eps=1e-3),      # no averaging at all
    dict(lr=1.0, beta1=0.5, beta2=0.25, eps=0.0),      # eps = 0: 0 / 0 is NaN where g = m = 0
    dict(lr=3e-4, beta1=0.95, beta2=0.98, eps=1e-6),
])
def test_hyperparameters_and_step_counts(zs, torch_mod, hp):
    """The step's constants as the kernel receives them, for several
    hyperparameter sets and step counts t = 1, 2, 1000, 2^40 (bias
    corrections from 1 - beta down to exactly 1): bit for bit with the
    oracle, NaN compared by class."""
    torch = torch_mod
    rng = np.random.default_rng(int(hp["lr"] * 1e4) + int(hp["beta1"] * 100))
    n = 20_011
    for t in (1, 2, 1000, 1 << 40):
        say(f"hyperparameters {hp} t={t}")
        g = (rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
        g[:7] = 0                                        # g = 0 rows (NaN when eps = 0 and m = v = 0)
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v0 = (rng.random(n) * 1e-6).astype(np.float32)
        m0[:3] = 0
        v0[:3] = 0
        host = HostShard(g.copy(), np.zeros(n, np.uint16), w0.copy(), m0.copy(), v0.copy())
        ref_flag = oracle.adam_step(host.g, host.p, host.w, host.m, host.v, t=t, **hp)
        dev = (torch.zeros(n, dtype=torch.float16, device="cuda"), to_dev16(g), to_dev32(w0),
               to_dev32(m0), to_dev32(v0))
        plan = zs.zero_plan_create([dev])
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        zs.zero_adam_step(plan, zs.AdamHParams(**hp), t, flag)
        torch.cuda.synchronize()
        assert _compare(dev, host, f"hp {hp} t={t}") == 0
        assert int(flag.item()) == ref_flag == 0
        plan.destroy()


@pytest.mark.parametrize("chunk", [0, 512])
def test_four_thousand_small_tensors(zs, torch_mod, chunk):
    """One plan over 4,000 tensors of 1 to 600 elements, each a view into
    five flat buffers at its own random gap (0-7 elements) in every buffer,
    so the five arrays of a tensor agree or disagree in alignment at random
    (vector path or single elements).  Two steps; the whole buffers are
    compared with the oracle applied tensor by tensor, and the gaps, filled
    with sentinels, must come back untouched."""
    torch = torch_mod
    rng = np.random.default_rng(4000 + chunk)
    T = 4000
    sizes = rng.integers(1, 601, T)
    offs = np.zeros((5, T), np.int64)
    ends = np.zeros(5, np.int64)
    for a in range(5):
        for k in range(T):
            offs[a, k] = ends[a] + rng.integers(0, 8)
            ends[a] = offs[a, k] + sizes[k]
    say(f"{T} small tensors chunk={chunk}: {int(sizes.sum())} elements")
    hp16 = np.full(ends[0] + 8, 0x7E01, np.uint16)                 # NaN sentinel in the gaps
    hg16 = np.full(ends[1] + 8, 0x3C00, np.uint16)
    hw = np.full(ends[2] + 8, 7.0, np.float32)
    hm = np.full(ends[3] + 8, -3.0, np.float32)
    hv = np.full(ends[4] + 8, 5.0, np.float32)
    for k in range(T):
        n = sizes[k]
        hw[offs[2, k]:offs[2, k] + n] = rng.standard_normal(n) * 0.02
        hm[offs[3, k]:offs[3, k] + n] = rng.standard_normal(n) * 1e-4
        hv[offs[4, k]:offs[4, k] + n] = rng.random(n) * 1e-6
    dp, dg, dw, dm, dv = to_dev16(hp16), to_dev16(hg16), to_dev32(hw), to_dev32(hm), to_dev32(hv)
    views = [(dp[offs[0, k]:offs[0, k] + sizes[k]], dg[offs[1, k]:offs[1, k] + sizes[k]],
              dw[offs[2, k]:offs[2, k] + sizes[k]], dm[offs[3, k]:offs[3, k] + sizes[k]],
              dv[offs[4, k]:offs[4, k] + sizes[k]]) for k in range(T)]
    plan = zs.zero_plan_create(views, chunk)
    st = plan.stats()
    assert st["n_tensors"] == T and st["n_params"] == int(sizes.sum())
    assert st["vector_elems"] and st["scalar_elems"]
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t in (3, 4):
        for k in range(T):
            n = sizes[k]
            hg16[offs[1, k]:offs[1, k] + n] = (rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
        dg.copy_(to_dev16(hg16))
        zs.zero_adam_step(plan, _hp(zs), t, flag)
        for k in range(T):
            n = sizes[k]
            sl = [slice(offs[a, k], offs[a, k] + n) for a in range(5)]
            oracle.adam_step(hg16[sl[1]], hp16[sl[0]], hw[sl[2]], hm[sl[3]], hv[sl[4]], t=t, **HP)
        torch.cuda.synchronize()
        assert np.array_equal(host16(dp), hp16), f"fp16 parameters differ at t={t}"
        for d, h, nm in ((dw, hw, "master"), (dm, hm, "m"), (dv, hv, "v")):
            assert np.array_equal(host32(d).view(np.uint32), h.view(np.uint32)), f"{nm} differs at t={t}"
    assert int(flag.item()) == 0
    plan.destroy()


def test_grid_at_its_limit_strides(zs, torch_mod):
    """A plan with more virtual workgroups than the largest grid: 2100 small
    tensors (1-299 elements, heads of 0-3) in 2^24-element chunks, 32,768
    tiles of 512 elements per chunk and almost all of them empty, so
    68,812,800 virtual workgroups on a grid of 2^26 - 1; the tensors from
    2048 on are reached only by striding.  One step, every element of the
    five buffers compared with the oracle (the gaps between tensors
    untouched)."""
    torch = torch_mod
    rng = np.random.default_rng(77)
    K = 2100
    sizes = rng.integers(1, 300, K)
    offs, pos = [], 0
    for k in range(K):
        pos += int(rng.integers(0, 4))
        offs.append(pos)
        pos += int(sizes[k])
    total = pos
    w0 = (rng.standard_normal(total) * 0.02).astype(np.float32)
    g = (rng.standard_normal(total) * 1e-3).astype(np.float16).view(np.uint16)
    dp = torch.zeros(total, dtype=torch.float16, device="cuda")
    dg = to_dev16(g)
    dw = to_dev32(w0)
    dm = torch.zeros(total, dtype=torch.float32, device="cuda")
    dv = torch.zeros(total, dtype=torch.float32, device="cuda")
    ents = [(dp[o:o + n], dg[o:o + n], dw[o:o + n], dm[o:o + n], dv[o:o + n])
            for o, n in zip(offs, sizes.tolist())]
    plan = zs.zero_plan_create(ents, 1 << 24)
    st = plan.stats()
    assert st["n_chunks"] == K and st["tile_elems"] == 512
    assert K * ((1 << 24) // 512) > (1 << 26) - 1
    say(f"grid limit: {K} tensors, {K * ((1 << 24) // 512)} virtual workgroups")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, _hp(zs), 1, flag)
    torch.cuda.synchronize()
    rp = np.zeros(total, np.uint16)
    rw, rm, rv = w0.copy(), np.zeros(total, np.float32), np.zeros(total, np.float32)
    rflag = 0
    for o, n in zip(offs, sizes.tolist()):
        rflag |= oracle.adam_step(g[o:o + n], rp[o:o + n], rw[o:o + n], rm[o:o + n],
                                  rv[o:o + n], t=1, **W.ADAM_HP)
    assert int(flag.item()) == rflag == 0
    res = [check16(host16(dp), rp, "grid limit param"), check32(host32(dw), rw, "grid limit master"),
           check32(host32(dm), rm, "grid limit m"), check32(host32(dv), rv, "grid limit v")]
    assert sum(r["not_bit_exact"] for r in res) == 0
    plan.destroy()
