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
    plan = zs.zero_plan_create([(p, g, w, m, v)])
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
