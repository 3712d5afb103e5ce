"""GPU parity of the bfloat16 variant (bfloat16 parameters and gradients,
fp32 master, m and v) through the C ABI, against the oracle's bfloat16 step
and reduce: ragged sizes at every alignment class, every bfloat16 gradient
pattern, the reduce over N_d from 1 to 64, the skip chain, and the full
7.5e9 / N_d = 64 rank's shard on sampled elements.  Each case prints its
name and sizes before it touches the GPU."""
import gc

import numpy as np
import pytest

import oracle
from parity import (check16, check32, check_whole16, check_whole32, host16, host32,
                    on_windows, to_dev32)
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


def to_devbf(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(x):
    return oracle.f32_to_bf16(np.asarray(x, np.float32))


def _step_ref(g, p, w, m, v, t):
    return oracle.adam_step(g, p, w, m, v, t=t, fmt="bf16", **HP)


def _cmp(dev, ref, what):
    p, w, m, v = dev
    P, Wr, M, V = ref
    res = [check16(host16(p), P, what + " param", fmt="bf16"), check32(host32(w), Wr, what + " master"),
           check32(host32(m), M, what + " m"), check32(host32(v), V, what + " v")]
    return sum(r["not_bit_exact"] for r in res)


SIZES = [1, 7, 8, 9, 31, 4095, 4096, 4097, 70001]
OFFSETS = [(0, 0, 0, 0, 0), (4, 0, 0, 0, 0), (3, 3, 3, 3, 3), (2, 6, 2, 2, 6),
           (1, 0, 0, 0, 0), (0, 0, 1, 0, 0)]


@pytest.mark.parametrize("chunk", [0, 512, "fine"])
def test_bf16_ragged_sizes_and_alignments(zs, chunk):
    """Tensors of sizes 1..70001 at every alignment class on 512-element
    tiles (chunk 0 or 512), and the same after one aligned tensor of 8M
    elements, which gives the plan 256-element tiles ("fine"); three steps,
    every element compared."""
    import torch
    fine = chunk == "fine"
    rng = np.random.default_rng(31 + (7 if fine else chunk))
    sizes_offs = [(n, OFFSETS[i % len(OFFSETS)]) for i, n in enumerate(SIZES)]
    if fine:
        sizes_offs = [(8 << 20, OFFSETS[0])] + sizes_offs
        chunk = 0
    dev, ref = [], []
    for n, offs in sizes_offs:
        bufs = [torch.zeros(n + o + 8, dtype=dt, device="cuda")[o:o + n] for o, dt in
                zip(offs, (torch.bfloat16, torch.bfloat16, torch.float32, torch.float32,
                           torch.float32))]
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v0 = (rng.random(n) * 1e-6).astype(np.float32)
        bufs[2].copy_(to_dev32(w0))
        bufs[3].copy_(to_dev32(m0))
        bufs[4].copy_(to_dev32(v0))
        dev.append(bufs)
        ref.append([np.zeros(n, np.uint16), w0.copy(), m0.copy(), v0.copy()])
    say(f"bf16 ragged chunk={chunk} fine={fine} tensors={len(dev)}")
    plan = zs.zero_plan_create([tuple(b) for b in dev], chunk)
    st = plan.stats()
    assert st["vector_elems"] and st["scalar_elems"]
    assert st["tile_elems"] == (256 if fine else 512)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    inexact = 0
    for t in (4, 5, 6):
        gs = []
        for b in dev:
            gh = bf16_bits(rng.standard_normal(b[2].numel()) * 1e-3)
            b[1].copy_(to_devbf(gh))
            gs.append(gh)
        zs.zero_adam_step(plan, zs.AdamHParams(**HP), t, flag)
        for gh, r in zip(gs, ref):
            _step_ref(gh, r[0], r[1], r[2], r[3], t)
        torch.cuda.synchronize()
        for k, (b, r) in enumerate(zip(dev, ref)):
            inexact += _cmp((b[0], b[2], b[3], b[4]), r, f"bf16 tensor {k} t={t}")
    assert int(flag.item()) == 0 and inexact == 0
    plan.destroy()


def test_bf16_every_gradient_pattern(zs):
    import torch
    n = 1 << 16
    say("bf16 every gradient pattern")
    rng = np.random.default_rng(8)
    g = np.arange(n, dtype=np.uint32).astype(np.uint16)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-6).astype(np.float32)
    dp = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    dw, dm, dv = to_dev32(w0), to_dev32(m0), to_dev32(v0)
    plan = zs.zero_plan_create([(dp, to_devbf(g), dw, dm, dv)])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 3, flag)
    ref = [np.zeros(n, np.uint16), w0.copy(), m0.copy(), v0.copy()]
    assert _step_ref(g, *ref, 3) == 1
    torch.cuda.synchronize()
    assert _cmp((dp, dw, dm, dv), ref, "bf16 all patterns") == 0
    assert int(flag.item()) == 1
    plan.destroy()


@pytest.mark.parametrize("nd", [1, 2, 3, 8, 16, 17, 64, 256])
@pytest.mark.parametrize("layout", ["aligned", "phase3", "mixed4h", "odd"])
def test_bf16_reduce_matches_oracle(zs, nd, layout):
    import torch
    rng = np.random.default_rng(100 + nd)
    for n in (1, 9, 1027, 4097, 65537):
        say(f"bf16 reduce nd={nd} layout={layout} n={n}")
        hs = [bf16_bits(rng.standard_normal(n) * 1e-3) for _ in range(nd)]
        offs = {"aligned": [0] * (nd + 1), "phase3": [3] * (nd + 1),
                "mixed4h": [1 + 4 * (r % 2) for r in range(nd + 1)],
                "odd": [r % 3 for r in range(nd + 1)]}[layout]
        ds = []
        for r in range(nd):
            b = torch.zeros(n + 8, dtype=torch.bfloat16, device="cuda")[offs[r]:offs[r] + n]
            b.copy_(to_devbf(hs[r]))
            ds.append(b)
        out = torch.zeros(n + 8, dtype=torch.bfloat16, device="cuda")[offs[nd]:offs[nd] + n]
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        zs.zero_reduce_grad_shard(ds, out, flag)
        ref, rflag = oracle.reduce_grad(hs, fmt="bf16")
        torch.cuda.synchronize()
        assert check16(host16(out), ref, f"bf16 reduce nd={nd} n={n}", fmt="bf16")["not_bit_exact"] == 0
        assert int(flag.item()) == rflag == 0


def test_bf16_reduce_then_step_skips_on_nonfinite(zs):
    """An infinite bfloat16 slice value raises the reduce's flag, which as
    the step's skip input leaves every array untouched."""
    import torch
    say("bf16 reduce -> skip")
    n = 5000
    rng = np.random.default_rng(3)
    hs = [bf16_bits(rng.standard_normal(n) * 1e-3) for _ in range(4)]
    hs[2][1234] = 0x7F80
    ds = [to_devbf(h) for h in hs]
    g = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    rflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_grad_shard(ds, g, rflag)
    p = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w, m, v = to_dev32(w0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    plan = zs.zero_plan_create([(p, g, w, m, v)])
    aflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1, aflag, rflag)
    torch.cuda.synchronize()
    assert int(rflag.item()) == 1 and int(aflag.item()) == 0
    assert np.array_equal(host32(w).view(np.uint32), w0.view(np.uint32))
    assert int(torch.count_nonzero(m).item()) == 0 and int(torch.count_nonzero(p).item()) == 0
    plan.destroy()


def test_bf16_flat_7p5b_nd64_full_size(zs):
    """Psi = 7.5e9 over 64 ranks, rank 0's 117,187,500 elements in bfloat16:
    reduce of 64 bfloat16 slices, then the step at t = 1; every element of
    the reduced gradient, param, master, m and v against the oracle's
    bfloat16 reduce and step on the same inputs (threaded over windows)."""
    import torch
    wl = W.WORKLOADS["flat_7p5b_nd64"]
    lay = zs.zero_shard_layout(wl.psi, wl.nd, 0, wl.align)
    n = lay.real_len
    say(f"bf16 flat_7p5b_nd64 n={n}")
    full, sh = W.device_flat_state(wl, lay.offset, n, lay.padded_total, half=torch.bfloat16)
    buf, rows = W.device_slices(wl, n, half=torch.bfloat16)
    w0 = host32(sh.w)
    slices = [host16(r) for r in rows]
    rflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    aflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_grad_shard(rows, sh.g, rflag)
    plan = zs.zero_plan_create([sh.arrays()])
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1, aflag, rflag)
    torch.cuda.synchronize()
    got_g = host16(sh.g)
    got = [host16(sh.p), host32(sh.w), host32(sh.m), host32(sh.v)]
    say("bf16 flat_7p5b_nd64: oracle over the whole shard")
    g_ref = np.empty(n, np.uint16)
    P, Wr = np.zeros(n, np.uint16), w0
    M, V = np.zeros(n, np.float32), np.zeros(n, np.float32)
    f1 = on_windows(lambda lo, hi: oracle.reduce_grad([x[lo:hi] for x in slices], g_ref[lo:hi],
                                                      fmt="bf16")[1], n)
    f2 = on_windows(lambda lo, hi: _step_ref(g_ref[lo:hi], P[lo:hi], Wr[lo:hi], M[lo:hi],
                                             V[lo:hi], 1), n)
    del slices
    res = [check_whole16(got_g, g_ref, "bf16 grad", fmt="bf16"),
           check_whole16(got[0], P, "bf16 param", fmt="bf16"),
           check_whole32(got[1], Wr, "bf16 master"), check_whole32(got[2], M, "bf16 m"),
           check_whole32(got[3], V, "bf16 v")]
    say(f"bf16 full size: all {n} elements, not bit-exact {[r['not_bit_exact'] for r in res]}")
    assert sum(r["not_bit_exact"] for r in res) == 0
    assert int(rflag.item()) == f1 == 0 and int(aflag.item()) == f2 == 0
    assert int(torch.count_nonzero(full[n:]).item()) == 0
    plan.destroy()
    del full, sh, buf, rows


# element offsets of ((even slices, odd slices), param, grad_out, master, m, v)
# inside their buffers, and the access path of the fused kernel each selects
FUSED_LAYOUTS = {
    "aligned": ((0, 0), 0, 0, 0, 0, 0),   # 16-byte slice loads, no head
    "phase2": ((2, 2), 2, 2, 2, 2, 2),    # 16-byte slice loads after a head of 6
    "split": ((0, 4), 0, 0, 0, 0, 0),     # slices agree only mod 8 bytes: 8-byte loads
    "odd": ((1, 1), 0, 0, 0, 0, 0),       # no common phase: single elements
}


def _fused_case(zs, n, nd, layout, with_gout, t, rng, inject=None):
    import torch
    so, po, go, wo, mo, vo = FUSED_LAYOUTS[layout]

    def view(off, dt):
        return torch.zeros(n + off + 8, dtype=dt, device="cuda")[off:off + n]

    hs = [bf16_bits(rng.standard_normal(n) * 1e-3) for _ in range(nd)]
    if inject is not None:
        r, i, bits = inject
        hs[r][i] = bits
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-6).astype(np.float32)
    ds = []
    for r in range(nd):
        b = view(so[r % 2], torch.bfloat16)
        b.copy_(to_devbf(hs[r]))
        ds.append(b)
    p = view(po, torch.bfloat16)
    gout = view(go, torch.bfloat16) if with_gout else None
    w, m, v = view(wo, torch.float32), view(mo, torch.float32), view(vo, torch.float32)
    w.copy_(to_dev32(w0))
    m.copy_(to_dev32(m0))
    v.copy_(to_dev32(v0))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_adam_step(ds, p, w, m, v, zs.AdamHParams(**HP), t, grad_out=gout,
                             nonfinite_flag=flag)
    g_ref, rflag = oracle.reduce_grad(hs, fmt="bf16")
    ref = (np.zeros(n, np.uint16), w0.copy(), m0.copy(), v0.copy())
    aflag = _step_ref(g_ref, *ref, t)
    torch.cuda.synchronize()
    what = f"bf16 fused n={n} nd={nd} {layout} gout={with_gout}"
    inexact = _cmp((p, w, m, v), ref, what)
    if with_gout:
        inexact += check16(host16(gout), g_ref, what + " grad", fmt="bf16")["not_bit_exact"]
    assert int(flag.item()) == (rflag | aflag)
    return inexact, rflag | aflag


@pytest.mark.parametrize("nd", [1, 3, 4, 8, 16, 17, 64, 256])
@pytest.mark.parametrize("layout", list(FUSED_LAYOUTS))
def test_bf16_fused_matches_oracle(zs, nd, layout):
    """The fused reduce + Adam step in bfloat16 against the oracle's
    bfloat16 reduce then its bfloat16 step: sizes from 1 to 70,001 (partial
    tiles, heads and tails), each access path, with and without the
    gradient output; every element."""
    rng = np.random.default_rng(8000 + nd)
    inexact = 0
    for n in (1, 5, 511, 512, 513, 70001):
        for with_gout in (False, True):
            say(f"bf16 fused nd={nd} layout={layout} n={n} gout={with_gout}")
            k, f = _fused_case(zs, n, nd, layout, with_gout, 3, rng)
            inexact += k
            assert f == 0
    assert inexact == 0, f"{inexact} elements within tolerance but not bit-exact"


@pytest.mark.parametrize("bits", [0x7F80, 0xFF80, 0x7FC0])
def test_bf16_fused_nonfinite(zs, bits):
    """An infinite or NaN bfloat16 slice value raises the flag and
    propagates per IEEE at its position only (the oracle decides which
    arrays turn non-finite)."""
    rng = np.random.default_rng(bits)
    say(f"bf16 fused inject {bits:#06x}")
    k, f = _fused_case(zs, 4099, 5, "aligned", True, 2, rng, inject=(3, 2050, bits))
    assert f == 1 and k == 0


def test_bf16_subnormal_masters_narrow_exactly(zs):
    """Masters at fp32 subnormals (and the first normals), g = 0 and m = v = 0
    at t = 1: the master is unchanged and the bfloat16 parameter is its
    round-to-nearest-even narrowing, subnormal results included (gfx950's
    conversion with denormals kept), bit for bit with the oracle."""
    import torch
    say("bf16 subnormal masters")
    n = 65_537
    rng = np.random.default_rng(16)
    b = rng.integers(1, 0x01000000, size=n, dtype=np.uint64).astype(np.uint32)
    b |= (rng.random(n) < 0.5).astype(np.uint32) << 31
    w0 = b.view(np.float32)
    g = np.zeros(n, np.uint16)
    P, Wr, M, V = np.zeros(n, np.uint16), w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    assert _step_ref(g, P, Wr, M, V, 1) == 0
    sub = (P & 0x7F80) == 0
    assert (sub & ((P & 0x7F) != 0)).sum() > 10000        # many subnormal bfloat16 results
    p = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    dev = (p, to_devbf(g), to_dev32(w0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda"))
    plan = zs.zero_plan_create([dev])
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1)
    torch.cuda.synchronize()
    assert _cmp((dev[0], dev[2], dev[3], dev[4]), (P, Wr, M, V), "bf16 subnormal masters") == 0
    plan.destroy()
