"""GPU parity of the Adam step, and of the fused reduce + Adam step, when
the 16-bit outputs (the parameter; the fused step's gradient output) are
out of phase with the other arrays (through the C ABI) against the CPU
oracle.

The parameter of a ZeRO shard is often a view of the full flattened
parameter buffer at the rank's offset, while the gradient, master, m and v
are the rank's own arrays; an offset that is not a multiple of four
elements puts the parameter 1-3 elements out of the others' 8-byte phase.
On tensors of 1,024 elements or more the library then keeps every other
array on the vector path and stores the parameter shifted: lanes hand
values to their neighbours so that the 8-byte stores are aligned, and the
few elements at each tile's edges go singly; the fused kernel below 16
slices does the same for both of its outputs.  Smaller tensors take single
elements throughout.  Tensors sit at element offsets that give every head
length class, with sizes around the head, the tile and the chunk
boundaries; every element is compared, and the parameter buffer outside
the views must stay untouched.  Each case prints its name before it
touches the GPU."""
import numpy as np
import pytest

import oracle
from parity import check16, check32, host16, host32, to_dev16, to_dev32
from test_gpu_tile_phase import Carved, _aligned, _head, _sizes
from zero_partitioned_mixed_layout_amd import workloads as W

pytestmark = pytest.mark.gpu
HP = dict(W.ADAM_HP)
OFFSETS = [0, 1, 2, 3, 64, 131, 253]


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


def _path(o, n):
    """(head, scalar elements) of a tensor at offset o whose parameter is
    out of phase: the vector path's head and singles from 1,024 elements,
    else every element singly (no head)."""
    if n < 1024:
        return 0, n
    h = _head(o, 0, n)
    singles = min(h % 4, n)
    return h, n - (n - singles) // 4 * 4


def _cases(fine):
    if not fine:
        return [(o, n) for o in OFFSETS for n in _sizes(_head(o, 0))]
    few = lambda h: sorted({x for x in (h + 1, h + 257, h + 1025, h + 16389) if x > 0})
    return [(0, 8 << 20)] + [(o, n) for o in OFFSETS for n in few(_head(o, 0))]


def _check_stats(st, cases):
    C = st["chunk_elems"]
    chunks = scalar = 0
    for o, n in cases:
        h, sc = _path(o, n)
        chunks += 1 + -(-(n - min(n, h + C)) // C)
        scalar += sc
    assert st["n_chunks"] == chunks
    assert st["scalar_elems"] == scalar
    assert st["vector_elems"] == sum(n for _, n in cases) - scalar


def _run_plan(zs, torch, c, plan, what, ls=None):
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = 0
    for t in (3, 4):
        zs.zero_adam_step(plan, zs.AdamHParams(**HP), t, flag, loss_scale=ls)
        c.oracle_step(t)
        torch.cuda.synchronize()
        bad += c.compare(f"{what} t={t}")
    assert int(flag.item()) == 0
    return bad


@pytest.mark.parametrize("chunk", [0, 512, "fine"])
@pytest.mark.parametrize("p_shift", [1, 2, 3])
def test_shifted_parameter_matches_oracle(zs, chunk, p_shift):
    """A plan over every offset and size with the parameter p_shift
    elements further into its buffer than the other arrays; the plan's
    counts show which tensors took the vector path; two steps.  chunk 512
    gives 512-element tiles; "fine" (one 8M-element tensor first) keeps the
    16,384-element chunk and the 256-element tile."""
    import torch
    fine = chunk == "fine"
    cases = _cases(fine)
    say(f"param shift: plan chunk={chunk} p_shift={p_shift} tensors={len(cases)}")
    c = Carved(torch, cases, 0, seed=500 + p_shift + (7 if fine else 0), p_shift=p_shift)
    plan = zs.zero_plan_create(c.tensors(), 0 if fine else chunk)
    st = plan.stats()
    if fine:
        assert st["tile_elems"] == 256 and st["chunk_elems"] == 16384
    elif chunk == 512:
        assert st["tile_elems"] == 512
    _check_stats(st, cases)
    bad = _run_plan(zs, torch, c, plan, f"plan chunk={chunk} p_shift={p_shift}")
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"
    plan.destroy()


@pytest.mark.parametrize("kind", ["bf16", "f16_scaled", "bf16_scaled"])
def test_shifted_parameter_other_formats(zs, kind):
    """bfloat16, and gradients that carry a loss scale of 2^12, with the
    parameter one element out of phase (the library's chunk)."""
    import torch
    fmt = "bf16" if kind.startswith("bf16") else "f16"
    k = 12 if kind.endswith("scaled") else None
    cases = _cases(False)
    say(f"param shift: {kind} tensors={len(cases)}")
    c = Carved(torch, cases, 0, seed=520 + len(kind), fmt=fmt, log2_scale=k, p_shift=1)
    plan = zs.zero_plan_create(c.tensors())
    _check_stats(plan.stats(), cases)
    ls = zs.LossScale(log2_scale=k, device=torch.device("cuda", 0)) if k is not None else None
    bad = _run_plan(zs, torch, c, plan, kind, ls)
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"
    plan.destroy()


@pytest.mark.parametrize("p_shift", [1, 3])
def test_shifted_parameter_noalloc(zs, p_shift):
    """The same tensors through the entry point that builds its chunk table
    in the library's fixed array; two steps."""
    import torch
    cases = _cases(False)
    say(f"param shift: noalloc p_shift={p_shift} tensors={len(cases)}")
    c = Carved(torch, cases, 0, seed=530 + p_shift, p_shift=p_shift)
    bad = 0
    for t in (3, 4):
        zs.zero_adam_step_noalloc(c.tensors(), zs.AdamHParams(**HP), t)
        c.oracle_step(t)
        torch.cuda.synchronize()
        bad += c.compare(f"noalloc p_shift={p_shift} t={t}")
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"


@pytest.mark.parametrize("p_shift", [1, 2, 3])
def test_shifted_parameter_split_route(zs, p_shift):
    """zero_reduce_adam_step at 32 slices with a gradient output (the
    reduce into it, then the one-tensor Adam kernel) and the parameter
    p_shift elements past the 1 KiB-aligned start of its buffer, the other
    arrays o elements past theirs; the bytes around the parameter view must
    stay untouched."""
    import torch
    nd = 32
    rng = np.random.default_rng(540 + p_shift)
    bad = 0
    for o in (0, 131):
        h = _head(o, 0)
        for n in sorted({1, 1023, 1024, h + 1025, h + 256 * 7 + 3, 70001, (1 << 20) + 5}):
            say(f"param shift: split route p_shift={p_shift} o={o} n={n} nd={nd}")
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
            pbuf = _aligned(torch, n + o + p_shift + 8, torch.float16)
            p = pbuf[o + p_shift:o + p_shift + n]
            gout = _aligned(torch, n + o, torch.float16)[o:]
            w, m, v = (_aligned(torch, n + o, torch.float32)[o:] for _ in range(3))
            w.copy_(to_dev32(w0))
            m.copy_(to_dev32(m0))
            v.copy_(to_dev32(v0))
            flag = torch.zeros(1, dtype=torch.int32, device="cuda")
            zs.zero_reduce_adam_step(ds, p, w, m, v, zs.AdamHParams(**HP), 3, grad_out=gout,
                                     nonfinite_flag=flag)
            g_ref, rflag = oracle.reduce_grad(hs)
            p_ref = np.zeros(n, np.uint16)
            aflag = oracle.adam_step(g_ref, p_ref, w0, m0, v0, t=3, **HP)
            torch.cuda.synchronize()
            hp_all = host16(pbuf)
            lo, hi = o + p_shift, o + p_shift + n
            assert not hp_all[:lo].any() and not hp_all[hi:].any(), \
                f"p_shift={p_shift} o={o} n={n}: bytes written outside the parameter view"
            what = f"split p_shift={p_shift} o={o} n={n}"
            r = [check16(hp_all[lo:hi], p_ref, what + " param"),
                 check16(host16(gout), g_ref, what + " grad"),
                 check32(host32(w), w0, what + " master"), check32(host32(m), m0, what + " m"),
                 check32(host32(v), v0, what + " v")]
            bad += sum(x["not_bit_exact"] for x in r)
            assert int(flag.item()) == (rflag | aflag)
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"


@pytest.mark.parametrize("chunk", [0, 512, "fine"])
@pytest.mark.parametrize("shifts", [(0, 1), (1, 1), (2, 3), (0, 2), (3, 1)])
def test_shifted_gradient_matches_oracle(zs, chunk, shifts):
    """The gradient (and in most cases the parameter too) out of the fp32
    arrays' phase, as views of full buffers at a rank's offset are: from
    1,024 elements the gradient's four values per lane come from two whole
    aligned 8-byte words joined in registers, and the parameter is stored
    shifted where it is out of phase as well; single elements below."""
    import torch
    ps, gs = shifts
    fine = chunk == "fine"
    cases = _cases(fine)
    say(f"param shift: plan chunk={chunk} p_shift={ps} g_shift={gs} tensors={len(cases)}")
    c = Carved(torch, cases, 0, seed=550 + 4 * ps + gs + (7 if fine else 0), p_shift=ps,
               g_shift=gs)
    plan = zs.zero_plan_create(c.tensors(), 0 if fine else chunk)
    st = plan.stats()
    if fine:
        assert st["tile_elems"] == 256 and st["chunk_elems"] == 16384
    _check_stats(st, cases)
    bad = _run_plan(zs, torch, c, plan, f"plan chunk={chunk} p_shift={ps} g_shift={gs}")
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"
    plan.destroy()


@pytest.mark.parametrize("kind", ["bf16", "f16_scaled", "bf16_scaled"])
def test_shifted_gradient_other_formats(zs, kind):
    """bfloat16 and loss-scaled gradients read shifted (gradient two
    elements, parameter one element out of phase)."""
    import torch
    fmt = "bf16" if kind.startswith("bf16") else "f16"
    k = 12 if kind.endswith("scaled") else None
    cases = _cases(False)
    say(f"param shift: gradient shifted, {kind} tensors={len(cases)}")
    c = Carved(torch, cases, 0, seed=570 + len(kind), fmt=fmt, log2_scale=k, p_shift=1,
               g_shift=2)
    plan = zs.zero_plan_create(c.tensors())
    _check_stats(plan.stats(), cases)
    ls = zs.LossScale(log2_scale=k, device=torch.device("cuda", 0)) if k is not None else None
    bad = _run_plan(zs, torch, c, plan, kind, ls)
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"
    plan.destroy()


@pytest.mark.parametrize("shifts", [(0, 3), (2, 1)])
def test_shifted_gradient_noalloc(zs, shifts):
    """The allocation-free entry point over tensors whose gradient is out of
    phase; two steps."""
    import torch
    ps, gs = shifts
    cases = _cases(False)
    say(f"param shift: noalloc p_shift={ps} g_shift={gs} tensors={len(cases)}")
    c = Carved(torch, cases, 0, seed=580 + 4 * ps + gs, p_shift=ps, g_shift=gs)
    bad = 0
    for t in (3, 4):
        zs.zero_adam_step_noalloc(c.tensors(), zs.AdamHParams(**HP), t)
        c.oracle_step(t)
        torch.cuda.synchronize()
        bad += c.compare(f"noalloc p_shift={ps} g_shift={gs} t={t}")
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"


@pytest.mark.parametrize("p_shift", [1, 2, 3])
@pytest.mark.parametrize("nd", [16, 32])
def test_shifted_parameter_split_route_in_place(zs, nd, p_shift):
    """zero_reduce_adam_step from 16 slices with no gradient output and the
    parameter out of the phase of the slices and the state: the reduce
    stores into the parameter view shifted, and the Adam step reads its
    gradient from there shifted and writes the new parameter in its place;
    the bytes around the view must stay untouched."""
    import torch
    rng = np.random.default_rng(590 + nd + p_shift)
    bad = 0
    for o in (0, 131):
        h = _head(o, 0)
        for n in sorted({5, 1023, 1024, h + 1025, h + 256 * 7 + 3, 70001, (1 << 20) + 5}):
            say(f"param shift: split route in place p_shift={p_shift} o={o} n={n} nd={nd}")
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
            pbuf = _aligned(torch, n + o + p_shift + 8, torch.float16)
            p = pbuf[o + p_shift:o + p_shift + n]
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
            hp_all = host16(pbuf)
            lo, hi = o + p_shift, o + p_shift + n
            assert not hp_all[:lo].any() and not hp_all[hi:].any(), \
                f"p_shift={p_shift} o={o} n={n}: bytes written outside the parameter view"
            what = f"split in place nd={nd} p_shift={p_shift} o={o} n={n}"
            r = [check16(hp_all[lo:hi], p_ref, what + " param"),
                 check32(host32(w), w0, what + " master"), check32(host32(m), m0, what + " m"),
                 check32(host32(v), v0, what + " v")]
            bad += sum(x["not_bit_exact"] for x in r)
            assert int(flag.item()) == (rflag | aflag)
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"


@pytest.mark.parametrize("o_shift", [1, 2, 3])
@pytest.mark.parametrize("slices", ["v16", "v8"])
@pytest.mark.parametrize("nd", [1, 4, 8, 16, 64])
def test_reduce_into_shifted_output(zs, nd, slices, o_shift):
    """zero_reduce_grad_shard into an output out of the slices' phase: the
    16-byte path ("v16") or the 8-byte path ("v8", slices four elements
    further) with the output stored shifted from 1,024 elements, single
    elements below; ragged sizes; bit-exact against the oracle, and the
    bytes around the output view untouched."""
    import torch
    so = 0 if slices == "v16" else 4
    rng = np.random.default_rng(700 + nd + so + o_shift)
    for n in (1000, 1024, 1029, 4096 + 259, 70001):
        say(f"param shift: reduce nd={nd} slices={slices} o_shift={o_shift} n={n}")
        hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
              for _ in range(nd)]
        ds = []
        for r in range(nd):
            b = _aligned(torch, n + so, torch.float16)[so:]
            b.copy_(to_dev16(hs[r]))
            ds.append(b)
        obuf = _aligned(torch, n + 8, torch.float16)
        out = obuf[o_shift:o_shift + n]
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        zs.zero_reduce_grad_shard(ds, out, nonfinite_flag=flag)
        g_ref, rflag = oracle.reduce_grad(hs)
        torch.cuda.synchronize()
        got = host16(obuf)
        what = f"reduce nd={nd} slices={slices} o_shift={o_shift} n={n}"
        assert not got[:o_shift].any() and not got[o_shift + n:].any(), what + ": guard"
        assert np.array_equal(got[o_shift:o_shift + n], g_ref), what
        assert int(flag.item()) == rflag


FUSED_OUTS = {"p1": (1, None), "p3": (3, None), "p2_g0": (2, 0), "p1_g1": (1, 1),
              "p3_g2": (3, 2), "p0_g1": (0, 1)}


@pytest.mark.parametrize("outs", list(FUSED_OUTS))
@pytest.mark.parametrize("slices", ["v16", "v8"])
@pytest.mark.parametrize("nd", [1, 3, 8, 12])
def test_shifted_outputs_fused_route(zs, nd, slices, outs):
    """zero_reduce_adam_step below 16 slices (one fused kernel) with the
    parameter, and the gradient output where there is one, out of the
    phase of the slices and the state: the fused kernel's 16-byte path
    (slices on 16 bytes, "v16") or 8-byte path ("v8", slices four elements
    further) with the outputs' stores shifted from 1,024 elements, single
    elements below; ragged sizes; the bytes around each output view must
    stay untouched."""
    import torch
    ps, gs = FUSED_OUTS[outs]
    so = 0 if slices == "v16" else 4
    rng = np.random.default_rng(600 + nd * 7 + so + ps * 3 + (gs or 0))
    bad = 0
    for n in (1000, 1029, 4096 + 259, 70001):
        say(f"param shift: fused route nd={nd} slices={slices} outs={outs} n={n}")
        hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
              for _ in range(nd)]
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v0 = (rng.random(n) * 1e-6).astype(np.float32)
        ds = []
        for r in range(nd):
            b = _aligned(torch, n + so, torch.float16)[so:]
            b.copy_(to_dev16(hs[r]))
            ds.append(b)
        pbuf = _aligned(torch, n + 8, torch.float16)
        p = pbuf[ps:ps + n]
        gbuf = _aligned(torch, n + 8, torch.float16) if gs is not None else None
        gout = gbuf[gs:gs + n] if gs is not None else None
        w, m, v = (_aligned(torch, n, torch.float32) for _ in range(3))
        w.copy_(to_dev32(w0))
        m.copy_(to_dev32(m0))
        v.copy_(to_dev32(v0))
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        zs.zero_reduce_adam_step(ds, p, w, m, v, zs.AdamHParams(**HP), 3, grad_out=gout,
                                 nonfinite_flag=flag)
        g_ref, rflag = oracle.reduce_grad(hs)
        p_ref = np.zeros(n, np.uint16)
        aflag = oracle.adam_step(g_ref, p_ref, w0, m0, v0, t=3, **HP)
        torch.cuda.synchronize()
        what = f"fused nd={nd} slices={slices} outs={outs} n={n}"
        hp_all = host16(pbuf)
        assert not hp_all[:ps].any() and not hp_all[ps + n:].any(), what + ": param guard"
        r = [check16(hp_all[ps:ps + n], p_ref, what + " param"),
             check32(host32(w), w0, what + " master"), check32(host32(m), m0, what + " m"),
             check32(host32(v), v0, what + " v")]
        if gs is not None:
            hg_all = host16(gbuf)
            assert not hg_all[:gs].any() and not hg_all[gs + n:].any(), what + ": grad guard"
            r.append(check16(hg_all[gs:gs + n], g_ref, what + " grad"))
        bad += sum(x["not_bit_exact"] for x in r)
        assert int(flag.item()) == (rflag | aflag)
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"


@pytest.mark.parametrize("route", ["fused_nd8_p1_g3", "split_nd32_in_place_p2", "reduce_nd16_o1",
                                   "reduce_nd4_v8_o3"])
def test_shifted_bfloat16_routes(zs, route):
    """The bfloat16 instantiations of the shifted stores and loads: the
    fused kernel (8 slices, parameter and gradient output out of phase), the
    split route in place (32 slices, no gradient output) and the reduce into
    a shifted output (16-byte and 8-byte paths); bit-exact against the
    oracle in bfloat16, the bytes around each written view untouched."""
    import torch
    kind, nd = route.split("_")[0], int(route.split("_")[1][2:])
    rng = np.random.default_rng(800 + len(route))
    for n in (1029, 4096 + 259, 70001):
        say(f"param shift: bf16 {route} n={n}")
        hs = [oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
              for _ in range(nd)]
        so = 4 if route.endswith("v8_o3") else 0
        ds = []
        for r in range(nd):
            b = _aligned(torch, n + so, torch.bfloat16)[so:]
            b.copy_(to_dev16(hs[r]).view(torch.bfloat16))
            ds.append(b)
        g_ref, rflag = oracle.reduce_grad(hs, fmt="bf16")
        what = f"bf16 {route} n={n}"
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        if kind == "reduce":
            os_ = int(route[-1])
            obuf = _aligned(torch, n + 8, torch.bfloat16)
            zs.zero_reduce_grad_shard(ds, obuf[os_:os_ + n], nonfinite_flag=flag)
            torch.cuda.synchronize()
            got = host16(obuf)
            assert not got[:os_].any() and not got[os_ + n:].any(), what + ": guard"
            assert np.array_equal(got[os_:os_ + n], g_ref), what
            assert int(flag.item()) == rflag
            continue
        ps = 1 if kind == "fused" else 2
        gs = 3 if kind == "fused" else None
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v0 = (rng.random(n) * 1e-6).astype(np.float32)
        pbuf = _aligned(torch, n + 8, torch.bfloat16)
        gbuf = _aligned(torch, n + 8, torch.bfloat16) if gs is not None else None
        w, m, v = (_aligned(torch, n, torch.float32) for _ in range(3))
        w.copy_(to_dev32(w0))
        m.copy_(to_dev32(m0))
        v.copy_(to_dev32(v0))
        zs.zero_reduce_adam_step(ds, pbuf[ps:ps + n], w, m, v, zs.AdamHParams(**HP), 3,
                                 grad_out=gbuf[gs:gs + n] if gs is not None else None,
                                 nonfinite_flag=flag)
        p_ref = np.zeros(n, np.uint16)
        aflag = oracle.adam_step(g_ref, p_ref, w0, m0, v0, t=3, fmt="bf16", **HP)
        torch.cuda.synchronize()
        hp_all = host16(pbuf)
        assert not hp_all[:ps].any() and not hp_all[ps + n:].any(), what + ": param guard"
        r = [check16(hp_all[ps:ps + n], p_ref, what + " param", fmt="bf16"),
             check32(host32(w), w0, what + " master"), check32(host32(m), m0, what + " m"),
             check32(host32(v), v0, what + " v")]
        if gs is not None:
            hg = host16(gbuf)
            assert not hg[:gs].any() and not hg[gs + n:].any(), what + ": grad guard"
            r.append(check16(hg[gs:gs + n], g_ref, what + " grad", fmt="bf16"))
        assert sum(x["not_bit_exact"] for x in r) == 0, what
        assert int(flag.item()) == (rflag | aflag)
