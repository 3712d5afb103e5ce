"""The step's entry points under HIP graph capture: neither the reduce nor
the Adam step allocates, synchronises or records a memset, so a caller can
capture a whole step (flag clear, reduce, Adam with the reduce's flag as
skip input) once and replay it.  The step number t is a host argument baked
into the captured launch, so every replay repeats the same t; the oracle
runs the same sequence.  Replays are interleaved with eager work and
synchronisations, and every replay is checked.  Each case prints its name
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


def test_captured_step_replays_match_the_oracle(zs):
    import torch
    n, nd, t = 70_001, 4, 3
    say(f"graph capture n={n} nd={nd}")
    rng = np.random.default_rng(12)
    hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16) for _ in range(nd)]
    slices = [to_dev16(h) for h in hs]
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = torch.empty(n, dtype=torch.float16, device="cuda")
    p = torch.zeros(n, dtype=torch.float16, device="cuda")
    w, m, v = to_dev32(w0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    rflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    aflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    # 16384-element chunks: this plan takes 256-element Adam tiles (the
    # loss-scaled test below takes 512)
    plan = zs.zero_plan_create([(p, g, w, m, v)], 16384)
    assert plan.stats()["tile_elems"] == 256
    hp = zs.AdamHParams(**HP)

    def step():
        rflag.zero_()   # a fill kernel, not a memset node
        zs.zero_reduce_grad_shard(slices, g, rflag)
        zs.zero_adam_step(plan, hp, t, aflag, rflag)

    # warm up on a side stream (as capture requires), then restore the state
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    w.copy_(to_dev32(w0))
    m.zero_()
    v.zero_()
    p.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    # capturing launched nothing: the state is still the initial one
    assert np.array_equal(host32(w).view(np.uint32), w0.view(np.uint32))
    g_ref, _ = oracle.reduce_grad(hs)
    P, Wr, M, V = np.zeros(n, np.uint16), w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for k in range(4):
        say(f"graph replay {k}")
        graph.replay()
        torch.cuda.synchronize()
        oracle.adam_step(g_ref, P, Wr, M, V, t=t, **HP)
        assert check16(host16(g), g_ref, "replay grad")["not_bit_exact"] == 0
        res = [check16(host16(p), P, "replay param"), check32(host32(w), Wr, "replay master"),
               check32(host32(m), M, "replay m"), check32(host32(v), V, "replay v")]
        assert sum(r["not_bit_exact"] for r in res) == 0, k
        assert int(rflag.item()) == 0 and int(aflag.item()) == 0
        # eager work between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        del scratch
    plan.destroy()


def test_captured_loss_scaled_step_follows_the_scale(zs):
    """reduce -> scaled Adam (skip = the reduce's flag) -> scale update,
    captured once and replayed six times with new slice contents written
    eagerly before each replay (infinities in replays 2 and 3).  The scale
    lives on the device, so replays read the scale the previous replay left:
    a skipped replay halves it and the next replays run with the new factor.
    No flag clear is captured: the update kernel clears the flag."""
    import torch
    n, nd, t = 40_003, 4, 2
    say(f"graph capture, loss-scaled step n={n} nd={nd}")
    rng = np.random.default_rng(13)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    slices = [torch.zeros(n, dtype=torch.float16, device="cuda") for _ in range(nd)]
    g = torch.empty(n, dtype=torch.float16, device="cuda")
    p = torch.zeros(n, dtype=torch.float16, device="cuda")
    w, m, v = to_dev32(w0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    rflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan = zs.zero_plan_create([(p, g, w, m, v)])
    assert plan.stats()["tile_elems"] == 512
    hp = zs.AdamHParams(**HP)
    ls = zs.LossScale(log2_scale=10, interval=2, min_log2=0, max_log2=12)
    init = ls.state.clone()

    def step():
        zs.zero_reduce_grad_shard(slices, g, rflag)
        zs.zero_adam_step(plan, hp, t, skip_if_nonzero=rflag, loss_scale=ls)
        ls.update(rflag)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    w.copy_(to_dev32(w0))
    m.zero_()
    v.zero_()
    p.zero_()
    ls.state.copy_(init)
    rflag.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    assert ls.read() == (10, 0, 0, 0)
    P, Wr, M, V = np.zeros(n, np.uint16), w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    st = (10, 0, 0, 0)
    for k in range(6):
        hs = [(rng.standard_normal(n) * 1e-3 * 2.0 ** st[0]).astype(np.float16).view(np.uint16)
              for _ in range(nd)]
        if k in (2, 3):
            hs[k][(k * 7919) % n] = 0xFC00
        for s_, h in zip(slices, hs):
            s_.copy_(to_dev16(h))
        torch.cuda.synchronize()
        say(f"graph replay {k} (scale 2^{st[0]})")
        graph.replay()
        torch.cuda.synchronize()
        g_ref, rf = oracle.reduce_grad(hs)
        assert rf == int(k in (2, 3))
        oracle.adam_step_scaled(g_ref, P, Wr, M, V, t=t, log2_scale=st[0], skip=bool(rf), **HP)
        st = oracle.loss_scale_update(st, rf, interval=2, min_log2=0, max_log2=12)
        assert ls.read() == st
        assert int(rflag.item()) == 0
        res = [check16(host16(p), P, "replay param"), check32(host32(w), Wr, "replay master"),
               check32(host32(m), M, "replay m"), check32(host32(v), V, "replay v")]
        assert sum(r["not_bit_exact"] for r in res) == 0, k
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        del scratch
    assert st[2] == 2 and st[3] == 4
    plan.destroy()


def test_captured_noalloc_step_rebuilds_its_table(zs):
    """zero_adam_step_noalloc captured with the reduce: the capture holds the
    launches that write the chunk table into the library's fixed array, so
    every replay rebuilds its own table.  Between replays an eager
    allocation-free step over other tensors overwrites that array; the next
    replay still matches the oracle.  Three tensors (views of one buffer
    each: ragged sizes, the third one's parameter one element off)."""
    import torch
    sizes, nd, t = (70_001, 513, 4099), 4, 2
    n = sum(sizes) + 8
    say(f"graph capture, allocation-free step, tensors {sizes}, nd={nd}")
    rng = np.random.default_rng(14)
    hs = [(rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16) for _ in range(nd)]
    slices = [to_dev16(h) for h in hs]
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = torch.empty(n, dtype=torch.float16, device="cuda")
    p = torch.zeros(n + 1, dtype=torch.float16, device="cuda")
    w, m, v = to_dev32(w0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    views, off = [], 0
    for k, s in enumerate(sizes):
        po = off + (1 if k == 2 else 0)
        views.append((p[po:po + s], g[off:off + s], w[off:off + s], m[off:off + s], v[off:off + s]))
        off += s + 2
    # another state whose eager steps overwrite the table between replays
    o = [torch.zeros(5000, dtype=torch.float16, device="cuda"), to_dev16(hs[0][:5000]),
         torch.ones(5000, device="cuda"), torch.zeros(5000, device="cuda"),
         torch.zeros(5000, device="cuda")]
    hp = zs.AdamHParams(**HP)

    def step():
        zs.zero_reduce_grad_shard(slices, g)
        zs.zero_adam_step_noalloc(views, hp, t)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    w.copy_(to_dev32(w0))
    m.zero_()
    v.zero_()
    p.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    assert np.array_equal(host32(w).view(np.uint32), w0.view(np.uint32))
    g_ref, _ = oracle.reduce_grad(hs)
    P, Wr = np.zeros(n + 1, np.uint16), w0.copy()
    M, V = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for k in range(4):
        say(f"graph replay {k}")
        graph.replay()
        torch.cuda.synchronize()
        off = 0
        for j, s in enumerate(sizes):
            po = off + (1 if j == 2 else 0)
            oracle.adam_step(g_ref[off:off + s], P[po:po + s], Wr[off:off + s], M[off:off + s],
                             V[off:off + s], t=t, **HP)
            off += s + 2
        res = [check16(host16(p), P, "replay param"), check32(host32(w), Wr, "replay master"),
               check32(host32(m), M, "replay m"), check32(host32(v), V, "replay v")]
        assert sum(r["not_bit_exact"] for r in res) == 0, k
        # an eager allocation-free step over other tensors rewrites the table
        zs.zero_adam_step_noalloc([tuple(o)], hp, k + 1)
        torch.cuda.synchronize()
