"""GPU parity of the fused stage-2 step (zero_reduce_adam_step) through the
C ABI.  Its definition is the reduce followed by the Adam step, so the
reference is the oracle's reduce_grad then adam_step on the same seeded
inputs; every element is compared.  At the full 7.5e9-parameter, N_d = 64
shard the fused kernel is also compared with the two separate kernels, bit
for bit over the whole arrays.  Each case prints its name and sizes before it
touches the GPU."""
import gc

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


def _view(torch, n, off, dtype):
    return torch.zeros(n + off + 8, dtype=dtype, device="cuda")[off:off + n]


# element offsets of ((even slices, odd slices), param, grad_out, master, m, v)
# inside their buffers, and the access path each selects
LAYOUTS = {
    "aligned": ((0, 0), 0, 0, 0, 0, 0),   # 16-byte slice loads, no head
    "phase2": ((2, 2), 2, 2, 2, 2, 2),    # 16-byte slice loads after a head of 6
    "mixed": ((4, 4), 0, 4, 0, 0, 0),     # 16-byte slice loads after a head of 4
    "split": ((0, 4), 0, 0, 0, 0, 0),     # slices agree only mod 8 bytes: 8-byte loads
    "odd": ((1, 1), 0, 0, 0, 0, 0),       # no common phase: single elements
    # parameter and gradient output one element off the state: the fused
    # kernel stores both shifted across lanes from 1,024 elements (single
    # elements below); from ZERO_FUSED_SPLIT_SLICES slices a single-element
    # reduce and the one-tensor Adam kernel's single path (its gradient,
    # the reduce's output, is off too)
    "param_off": ((0, 0), 1, 1, 0, 0, 0),
}


def _run_case(zs, torch, n, nd, layout, with_gout, t, rng, warm=True):
    so, po, go, wo, mo, vo = LAYOUTS[layout]
    hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16) for _ in range(nd)]
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32) if warm else np.zeros(n, np.float32)
    v0 = (rng.random(n) * 1e-6).astype(np.float32) if warm else np.zeros(n, np.float32)
    ds = []
    for r in range(nd):
        b = _view(torch, n, so[r % 2], torch.float16)
        b.copy_(to_dev16(hs[r]))
        ds.append(b)
    p = _view(torch, n, po, torch.float16)
    gout = _view(torch, n, go, torch.float16) if with_gout else None
    w = _view(torch, n, wo, torch.float32)
    m = _view(torch, n, mo, torch.float32)
    v = _view(torch, n, vo, torch.float32)
    w.copy_(to_dev32(w0))
    m.copy_(to_dev32(m0))
    v.copy_(to_dev32(v0))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_adam_step(ds, p, w, m, v, zs.AdamHParams(**HP), t, grad_out=gout,
                             nonfinite_flag=flag)
    g_ref, rflag = oracle.reduce_grad(hs)
    p_ref = np.zeros(n, np.uint16)
    w_ref, m_ref, v_ref = w0.copy(), m0.copy(), v0.copy()
    aflag = oracle.adam_step(g_ref, p_ref, w_ref, m_ref, v_ref, t=t, **HP)
    torch.cuda.synchronize()
    what = f"fused n={n} nd={nd} {layout} gout={with_gout}"
    res = [check16(host16(p), p_ref, what + " param"), check32(host32(w), w_ref, what + " master"),
           check32(host32(m), m_ref, what + " m"), check32(host32(v), v_ref, what + " v")]
    if with_gout:
        res.append(check16(host16(gout), g_ref, what + " grad"))
    assert int(flag.item()) == (rflag | aflag)
    return sum(r["not_bit_exact"] for r in res)


@pytest.mark.parametrize("nd", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 31, 32, 33, 64, 256])
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_fused_matches_oracle(zs, nd, layout):
    """Sizes from 1 to 70,001 (partial tiles, heads and tails), each access
    path, with and without the fp16 gradient output; every element."""
    import torch
    rng = np.random.default_rng(7000 + nd)
    inexact = 0
    for n in (1, 3, 4, 5, 511, 512, 513, 1029, 70001):
        for with_gout in (False, True):
            say(f"fused nd={nd} layout={layout} n={n} gout={with_gout}")
            inexact += _run_case(zs, torch, n, nd, layout, with_gout, t=3, rng=rng)
    assert inexact == 0, f"{inexact} elements within tolerance but not bit-exact"


def test_fused_first_step_and_zero_size(zs):
    """t = 1 from m = v = 0; n = 0 launches nothing and leaves the flag."""
    import torch
    rng = np.random.default_rng(11)
    say("fused t=1 n=4097 nd=8")
    assert _run_case(zs, torch, 4097, 8, "aligned", True, t=1, rng=rng, warm=False) == 0
    say("fused n=0")
    e = torch.zeros(0, dtype=torch.float16, device="cuda")
    e32 = torch.zeros(0, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_adam_step([e, e.clone()], e.clone(), e32, e32.clone(), e32.clone(),
                             zs.AdamHParams(**HP), 1, nonfinite_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0


def test_fused_special_values(zs):
    """Every fp16 bit pattern as the single slice (N_d = 1), then slices
    whose mean overflows or meets +inf with -inf: IEEE classes in param,
    master, m, v and the gradient output match the oracle, and the flag is
    raised."""
    import torch
    say("fused special: all 65,536 patterns, nd=1")
    n = 1 << 16
    bits = np.arange(n, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(5)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p = torch.zeros(n, dtype=torch.float16, device="cuda")
    gout = torch.zeros(n, dtype=torch.float16, device="cuda")
    w, m, v = to_dev32(w0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_adam_step([to_dev16(bits)], p, w, m, v, zs.AdamHParams(**HP), 1,
                             grad_out=gout, nonfinite_flag=flag)
    g_ref, rflag = oracle.reduce_grad([bits])
    p_ref, w_ref = np.zeros(n, np.uint16), w0.copy()
    m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32)
    aflag = oracle.adam_step(g_ref, p_ref, w_ref, m_ref, v_ref, t=1, **HP)
    torch.cuda.synchronize()
    check16(host16(gout), g_ref, "all patterns grad")
    check16(host16(p), p_ref, "all patterns param")
    for got, ref, nm in ((w, w_ref, "master"), (m, m_ref, "m"), (v, v_ref, "v")):
        check32(host32(got), ref, "all patterns " + nm)
    assert int(flag.item()) == (rflag | aflag) == 1

    say("fused special: overflow and inf-inf, nd=3")
    a = np.array([0x7BFF, 0x7C00, 0xFC00, 0x3C00, 0x0001, 0x7E00] * 200, np.uint16)
    b = np.array([0x7BFF, 0xFC00, 0x3C00, 0x3C00, 0x8001, 0x3C00] * 200, np.uint16)
    c = np.array([0x7BFF, 0x3C00, 0x7C00, 0xBC00, 0x0000, 0x3C00] * 200, np.uint16)
    k = a.size
    w0 = (rng.standard_normal(k) * 0.02).astype(np.float32)
    p = torch.zeros(k, dtype=torch.float16, device="cuda")
    w, m, v = to_dev32(w0), torch.zeros(k, device="cuda"), torch.zeros(k, device="cuda")
    flag.zero_()
    zs.zero_reduce_adam_step([to_dev16(a), to_dev16(b), to_dev16(c)], p, w, m, v,
                             zs.AdamHParams(**HP), 2, nonfinite_flag=flag)
    g_ref, rflag = oracle.reduce_grad([a, b, c])
    p_ref, w_ref = np.zeros(k, np.uint16), w0.copy()
    m_ref, v_ref = np.zeros(k, np.float32), np.zeros(k, np.float32)
    aflag = oracle.adam_step(g_ref, p_ref, w_ref, m_ref, v_ref, t=2, **HP)
    torch.cuda.synchronize()
    check16(host16(p), p_ref, "overflow param")
    for got, ref, nm in ((w, w_ref, "master"), (m, m_ref, "m"), (v, v_ref, "v")):
        check32(host32(got), ref, "overflow " + nm)
    assert int(flag.item()) == (rflag | aflag) == 1


def test_fused_rejects_through_binding(zs):
    """Overlapping written arrays and bad sizes are refused before launch."""
    import torch
    say("fused rejects")
    s = torch.zeros(64, dtype=torch.float16, device="cuda")
    p = torch.zeros(64, dtype=torch.float16, device="cuda")
    w = torch.zeros(64, device="cuda")
    m, v = torch.zeros(64, device="cuda"), torch.zeros(64, device="cuda")
    hp = zs.AdamHParams(**HP)
    with pytest.raises(zs.ZeroError):        # param is one of the slices
        zs.zero_reduce_adam_step([s, p], p, w, m, v, hp, 1)
    with pytest.raises(zs.ZeroError):        # m and v the same array
        zs.zero_reduce_adam_step([s], p, w, m, m, hp, 1)
    with pytest.raises(zs.ZeroError):        # grad_out overlaps the param
        zs.zero_reduce_adam_step([s], p, w, m, v, hp, 1, grad_out=p)
    with pytest.raises(zs.ZeroError):        # t = 0
        zs.zero_reduce_adam_step([s], p, w, m, v, hp, 0)
    with pytest.raises(ValueError):          # sizes differ
        zs.zero_reduce_adam_step([s[:32]], p, w, m, v, hp, 1)
    # two ranks may hand in the same read-only slice
    zs.zero_reduce_adam_step([s, s], p, w, m, v, hp, 1)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["flat_7p5b_nd64", "flat_7p5b_nd8"])
def test_fused_equals_separate_kernels_at_full_size(zs, name):
    """Psi = 7.5e9 over 64 ranks (rank 0's 117,187,500 elements, 64 slices:
    the state loaded before the slices) and over 8 ranks (rank 3's
    937,500,160 elements, 8 slices: the state loaded after them), as bench.py
    times them with --fused: the fused kernel against zero_reduce_grad_shard
    + zero_adam_step on identical copies of the state, every element of
    every array bit for bit; sampled elements also against the oracle."""
    import torch
    wl = W.WORKLOADS[name]
    lay = zs.zero_shard_layout(wl.psi, wl.nd, wl.rank, wl.align)
    n = lay.real_len
    say(f"fused full size n={n} nd={wl.nd}")
    full, sh = W.device_flat_state(wl, lay.offset, n, lay.padded_total)
    buf, rows = W.device_slices(wl, n)
    # second copy of the state for the separate kernels
    w2, m2, v2 = sh.w.clone(), sh.m.clone(), sh.v.clone()
    p2 = torch.zeros(n, dtype=torch.float16, device="cuda")
    g2 = torch.zeros(n, dtype=torch.float16, device="cuda")
    idx = W.sample_indices(n, 100_000, seed=wl.seed + 99)
    d = torch.from_numpy(idx).cuda()
    w0 = host32(sh.w.index_select(0, d))
    slices = [host16(r.index_select(0, d)) for r in rows]
    hp = zs.AdamHParams(**HP)
    f1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    f2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    gout = torch.zeros(n, dtype=torch.float16, device="cuda")
    zs.zero_reduce_adam_step(rows, sh.p, sh.w, sh.m, sh.v, hp, 1, grad_out=gout, nonfinite_flag=f1)
    zs.zero_reduce_grad_shard(rows, g2, f2)
    plan = zs.zero_plan_create([(p2, g2, w2, m2, v2)])
    zs.zero_adam_step(plan, hp, 1, f2)
    torch.cuda.synchronize()
    for a, b, nm in ((sh.p, p2, "param"), (gout, g2, "grad")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), nm
    for a, b, nm in ((sh.w, w2, "master"), (sh.m, m2, "m"), (sh.v, v2, "v")):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), nm
    assert int(f1.item()) == int(f2.item()) == 0
    g_ref, _ = oracle.reduce_grad(slices)
    p_ref = np.zeros(idx.size, np.uint16)
    m_ref = np.zeros(idx.size, np.float32)
    v_ref = np.zeros(idx.size, np.float32)
    w_ref = w0.copy()
    oracle.adam_step(g_ref, p_ref, w_ref, m_ref, v_ref, t=1, **HP)
    res = [check16(host16(sh.p.index_select(0, d)), p_ref, "full param"),
           check32(host32(sh.w.index_select(0, d)), w_ref, "full master"),
           check32(host32(sh.m.index_select(0, d)), m_ref, "full m"),
           check32(host32(sh.v.index_select(0, d)), v_ref, "full v")]
    assert sum(r["not_bit_exact"] for r in res) == 0
    # other ranks' part of the full fp16 parameter buffer is untouched
    assert int(torch.count_nonzero(full[:lay.offset]).item()) == 0
    assert int(torch.count_nonzero(full[lay.offset + n:]).item()) == 0
    plan.destroy()
    del full, sh, buf, rows, w2, m2, v2, p2, g2, gout
    gc.collect()
    torch.cuda.empty_cache()
