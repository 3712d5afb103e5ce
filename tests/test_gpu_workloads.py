"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same entry points, same plans).

The flat shards (117,187,500 and 937,500,160 elements) are compared with
the oracle element by element over their whole arrays: the oracle runs
from the same seeded inputs -- the initial master, every slice and every
step's gradients copied to the host before the GPU uses them, never a value
the HIP path produced -- through all warm-up steps, threaded over windows
of the arrays on the host's CPUs.  The tensor lists (GPT-2-XL, Llama-7B)
are compared through their six steps at sampled elements (both ends of
every tensor and 96 random ones): their whole state with every step's
gradients would pass the host memory a GPU job may use (about 280 GB for
Llama-7B).  The Llama-7B list is also compared over its whole arrays for
its first step from the seeded state (about 108 GB of host memory).
Properties that hold at any size (untouched padding and other ranks'
parameters, the non-finite positions, the ZeRO-2 ledger) are checked on
the whole arrays."""
import gc

import numpy as np
import pytest

import oracle
from parity import (check16, check32, check_whole16, check_whole32, host16, host32,
                    host_threads, on_windows)
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


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    import torch
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def _gather16(t, idx_dev):
    return host16(t.index_select(0, idx_dev))


def _gather32(t, idx_dev):
    return host32(t.index_select(0, idx_dev))


def _oracle_steps(w0, grads_by_step, t0=1):
    n = w0.size
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p = np.zeros(n, np.uint16)
    flag = 0
    for k, g in enumerate(grads_by_step):
        flag |= oracle.adam_step(g, p, w, m, v, t=t0 + k, **HP)
    return p, w, m, v, flag


def _check_whole(got, ref, what):
    p, w, m, v = got
    rp, rw, rm, rv = ref
    res = [check_whole16(p, rp, f"{what} param"), check_whole32(w, rw, f"{what} master"),
           check_whole32(m, rm, f"{what} m"), check_whole32(v, rv, f"{what} v")]
    inexact = sum(r["not_bit_exact"] for r in res)
    say(f"{what}: all {res[0]['n']} elements, max rel "
        f"{max(r.get('max_rel', 0) for r in res):.2g}, not bit-exact {inexact}, "
        f"bit patterns differing (NaN payloads included) {[r['bits_differ'] for r in res]}")
    return inexact


def _check_all(got, ref, what):
    p, w, m, v = got
    rp, rw, rm, rv = ref
    res = [check16(p, rp, f"{what} param"), check32(w, rw, f"{what} master"),
           check32(m, rm, f"{what} m"), check32(v, rv, f"{what} v")]
    inexact = sum(r["not_bit_exact"] for r in res)
    say(f"{what}: {res[0]['n']} sampled elements, max rel "
        f"{max(r.get('max_rel', 0) for r in res):.2g}, not bit-exact {inexact}")
    return inexact


@pytest.mark.parametrize("name,layout", [("gpt2_xl", "flat"), ("gpt2_xl", "separate"),
                                         ("llama_7b", "flat"), ("llama_7b", "separate")])
def test_tensor_list_workload(zs, name, layout):
    """GPT-2-XL (580 tensors, 1.56e9 params) and Llama-7B (291 tensors,
    6.74e9 params, 108 GB of state in HBM): 5 warm-up steps, then step 6,
    one plan over the whole list, N_d = 1.  Both caller layouts: views into
    five flattened buffers, and five allocations per tensor."""
    import torch
    wl = W.WORKLOADS[name]
    say(f"{name} ({layout}): {len(wl.tensors)} tensors, {wl.n_params} params")
    assert zs.zero_state_bytes(0, wl.n_params, 1) == 16 * wl.n_params
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    tensors = W.device_list_state(wl, layout=layout)
    torch.cuda.synchronize()
    held = torch.cuda.memory_allocated() - before
    if layout == "flat":
        assert tensors[1].w.data_ptr() == tensors[0].w.data_ptr() + 4 * tensors[0].n
    if layout == "flat":
        # the stage-0 ledger, 16 bytes per parameter, against what the
        # allocator holds for the five buffers (torch hands out large blocks
        # in 2 MiB segments: under 2 MiB of rounding each)
        assert 0 <= held - 16 * wl.n_params < 5 * (2 << 20), (held, 16 * wl.n_params)
    plan = zs.zero_plan_create([t.arrays() for t in tensors])
    st = plan.stats()
    assert st["n_params"] == wl.n_params and st["vector_elems"] == wl.n_params
    idx = [W.sample_indices(t.n, 96, seed=wl.seed + 13 * k) for k, t in enumerate(tensors)]
    idx_dev = [torch.from_numpy(i).cuda() for i in idx]
    w0 = np.concatenate([_gather32(t.w, d) for t, d in zip(tensors, idx_dev)])
    grads = []
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp = zs.AdamHParams(**HP)
    for t in range(1, wl.warm_steps + 2):
        W.device_fill_grads(wl, tensors, t)
        grads.append(np.concatenate([_gather16(x.g, d) for x, d in zip(tensors, idx_dev)]))
        say(f"{name}: step t={t}")
        zs.zero_adam_step(plan, hp, t, flag)
    torch.cuda.synchronize()
    got = [np.concatenate([f(getattr(x, a), d) for x, d in zip(tensors, idx_dev)])
           for a, f in (("p", _gather16), ("w", _gather32), ("m", _gather32), ("v", _gather32))]
    rp, rw, rm, rv, rflag = _oracle_steps(w0, grads)
    assert int(flag.item()) == rflag == 0
    assert _check_all(got, (rp, rw, rm, rv), name) == 0
    plan.destroy()


@pytest.mark.parametrize("rank", [0, 1, 63])
def test_flat_7p5b_nd64_reduce_then_step(zs, rank):
    """Psi = 7.5e9 over 64 ranks: this rank's 117,187,500-element partition.
    64 fp16 gradient slices are averaged, then Adam runs at t = 1 with the
    reduce's flag as its skip input.  Odd ranks' fp16 parameter views start
    8 bytes off a 16-byte boundary (still the vector path, whose fp16
    accesses are 8 bytes wide).  Every element of the reduced gradient,
    param, master, m and v is compared with the oracle.  The whole
    other-rank part of the fp16 parameter buffer stays untouched, and the
    allocated ZeRO-2 state equals the ledger's 16,640,625,000 bytes."""
    import torch
    wl = W.WORKLOADS["flat_7p5b_nd64"]
    lay = zs.zero_shard_layout(wl.psi, wl.nd, rank, wl.align)
    assert lay._asdict() == oracle.shard_layout(wl.psi, wl.nd, rank, wl.align)
    n = lay.real_len
    say(f"flat_7p5b_nd64 rank={rank} n={n} offset={lay.offset}")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    full, sh = W.device_flat_state(wl, lay.offset, n, lay.padded_total)
    torch.cuda.synchronize()
    held = torch.cuda.memory_allocated() - before     # what the allocator holds for the state
    buf, rows = W.device_slices(wl, n)
    ledger = full.numel() * 2 + sh.g.numel() * 2 + 3 * 4 * sh.w.numel()
    assert ledger == zs.zero_state_bytes(2, wl.psi, wl.nd, wl.align) == 16_640_625_000
    # five allocations, each rounded up by under 2 MiB (the allocator's
    # segment size for large blocks)
    assert 0 <= held - ledger < 5 * (2 << 20), (held, ledger)
    plan = zs.zero_plan_create([sh.arrays()])
    st = plan.stats()
    assert st["vector_elems"] >= n - 3
    # the oracle's inputs, copied before the GPU step
    w0 = host32(sh.w)
    slices = [host16(r) for r in rows]
    rflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    aflag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_reduce_grad_shard(rows, sh.g, rflag)
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1, aflag, rflag)
    torch.cuda.synchronize()
    got_g = host16(sh.g)
    got = [host16(sh.p), host32(sh.w), host32(sh.m), host32(sh.v)]
    say(f"flat_7p5b_nd64 rank={rank}: oracle over the whole shard on {host_threads()} threads")
    g_ref = np.empty(n, np.uint16)
    rp, rw = np.zeros(n, np.uint16), w0
    rm, rv = np.zeros(n, np.float32), np.zeros(n, np.float32)
    fr = on_windows(lambda lo, hi: oracle.reduce_grad([x[lo:hi] for x in slices],
                                                       g_ref[lo:hi])[1], n)
    fa = on_windows(lambda lo, hi: oracle.adam_step(g_ref[lo:hi], rp[lo:hi], rw[lo:hi],
                                                     rm[lo:hi], rv[lo:hi], t=1, **HP), n)
    del slices
    r = check_whole16(got_g, g_ref, "reduced gradient")
    say(f"reduced gradient: all {n} elements, not bit-exact {r['not_bit_exact']}")
    assert r["not_bit_exact"] == 0 and int(rflag.item()) == fr == 0
    assert _check_whole(got, (rp, rw, rm, rv), f"nd64 rank {rank}") == 0
    assert int(aflag.item()) == fa == 0
    before = int(torch.count_nonzero(full[:lay.offset]).item())
    after = int(torch.count_nonzero(full[lay.offset + n:]).item())
    assert before == after == 0
    plan.destroy()


def test_flat_7p5b_nd8_rank3_with_infinities(zs):
    """Psi = 7.5e9 over 8 ranks in 512-element units: rank 3's 937,500,160
    elements at 2,812,500,480.  Five warm-up steps with finite gradients,
    then step 6 with 93,750 (0.01%) gradients set to +-inf: the flag is 1,
    and master, m, v and fp16 param are non-finite exactly there.  Every
    element of param, master, m and v after step 6 is compared with the
    oracle run through all six steps."""
    import torch
    wl = W.WORKLOADS["flat_7p5b_nd8"]
    lay = zs.zero_shard_layout(wl.psi, wl.nd, wl.rank, wl.align)
    assert lay._asdict() == oracle.shard_layout(wl.psi, wl.nd, wl.rank, wl.align)
    assert (lay.shard_len, lay.offset, lay.real_len) == (937_500_160, 2_812_500_480, 937_500_160)
    n = lay.real_len
    say(f"flat_7p5b_nd8 rank 3 n={n}")
    full, sh = W.device_flat_state(wl, lay.offset, n, lay.padded_total)
    plan = zs.zero_plan_create([sh.arrays()])
    pos, sign = W.inf_positions(n, wl.inf_frac, wl.seed)
    assert pos.size == 93_750
    w0 = host32(sh.w)
    grads = []
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp = zs.AdamHParams(**HP)
    T = wl.warm_steps + 1
    for t in range(1, T + 1):
        W.device_fill_grads(wl, [sh], t)
        if t == T:
            W.device_inject_inf(sh.g, pos, sign)
            torch.cuda.synchronize()
            assert int(flag.item()) == 0          # warm-up steps were finite
        grads.append(host16(sh.g))
        say(f"flat_7p5b_nd8: step t={t}")
        zs.zero_adam_step(plan, hp, t, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    got = [host16(sh.p), host32(sh.w), host32(sh.m), host32(sh.v)]
    rp, rw = np.zeros(n, np.uint16), w0
    rm, rv = np.zeros(n, np.float32), np.zeros(n, np.float32)
    rflag = 0
    for t, g in enumerate(grads, start=1):
        say(f"flat_7p5b_nd8: oracle step t={t} over the whole shard on {host_threads()} threads")
        rflag |= on_windows(lambda lo, hi: oracle.adam_step(g[lo:hi], rp[lo:hi], rw[lo:hi],
                                                             rm[lo:hi], rv[lo:hi], t=t, **HP), n)
        assert rflag == (1 if t == T else 0)
    del grads
    assert _check_whole(got, (rp, rw, rm, rv), "nd8 rank 3") == 0
    # whole arrays: non-finite exactly at the injected positions
    pos_dev = torch.from_numpy(pos).cuda()
    for a in (sh.w, sh.p):
        bad = torch.nonzero(~torch.isfinite(a)).flatten()
        assert torch.equal(bad, pos_dev)
    bad_m = torch.nonzero(~torch.isfinite(sh.m)).flatten()
    assert torch.equal(bad_m, pos_dev)
    assert int(torch.count_nonzero(full[:lay.offset]).item()) == 0
    assert int(torch.count_nonzero(full[lay.offset + n:]).item()) == 0
    plan.destroy()


def _host_bytes_free() -> int:
    """Host memory this process may still take: the kernel's MemAvailable,
    capped by the cgroup's limit less its current use where one is set."""
    free = 0
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemAvailable:"):
                free = int(line.split()[1]) * 1024
    except OSError:
        return 0
    try:
        lim = open("/sys/fs/cgroup/memory.max").read().strip()
        if lim != "max":
            used = int(open("/sys/fs/cgroup/memory.current").read())
            free = min(free, int(lim) - used)
    except (OSError, ValueError):
        pass
    return free


def test_llama_7b_whole_arrays_first_step(zs):
    """The Llama-7B list (291 tensors, 6,738,415,616 parameters) in five
    flattened buffers: step 1 from the seeded state (master N(0, 0.02),
    m = v = 0; master and the step's gradients copied to the host before the
    GPU uses them), every element of the parameter, master, m and v
    compared with the oracle.  The step is elementwise with one set of
    hyperparameters, so the oracle over the flattened arrays in windows is
    the step of every tensor.  test_tensor_list_workload follows the
    workload's six steps at sampled elements.  Skipped where the host
    cannot hold the state (16 bytes per parameter, about 108 GB)."""
    import torch
    wl = W.WORKLOADS["llama_7b"]
    N = wl.n_params
    need = 16 * N + (8 << 30)
    if _host_bytes_free() < need:
        pytest.skip(f"needs about {need >> 30} GiB of host memory, "
                    f"{_host_bytes_free() >> 30} GiB free")
    say(f"llama_7b whole arrays: {len(wl.tensors)} tensors, {N} params")
    tensors = W.device_list_state(wl, layout="flat")
    W.device_fill_grads(wl, tensors, 1)
    torch.cuda.synchronize()
    bp, bg, bw, bm, bv = (getattr(tensors[0], a)._base for a in "pgwmv")
    for b in (bp, bg, bw, bm, bv):
        assert b is not None and b.numel() == N
    say("llama_7b: seeded state and gradients to the host")
    g, w, m, v = host16(bg), host32(bw), host32(bm), host32(bv)
    assert not np.any(m) and not np.any(v)
    p = np.zeros(N, np.uint16)
    plan = zs.zero_plan_create([t.arrays() for t in tensors])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1, flag)
    torch.cuda.synchronize()
    blocks, rflag = 24, 0
    for b in range(blocks):
        lo, hi = N * b // blocks, N * (b + 1) // blocks

        def step(a, z, lo=lo):
            return oracle.adam_step(g[lo + a:lo + z], p[lo + a:lo + z], w[lo + a:lo + z],
                                    m[lo + a:lo + z], v[lo + a:lo + z], t=1, **HP)

        rflag |= on_windows(step, hi - lo)
        say(f"llama_7b: oracle block {b + 1}/{blocks}")
    bad, win = 0, 1 << 28
    for lo in range(0, N, win):
        hi = min(N, lo + win)
        got = (host16(bp[lo:hi]), host32(bw[lo:hi]), host32(bm[lo:hi]), host32(bv[lo:hi]))
        bad += _check_whole(got, (p[lo:hi], w[lo:hi], m[lo:hi], v[lo:hi]),
                            f"llama_7b [{lo}, {hi})")
    assert int(flag.item()) == rflag == 0
    assert bad == 0, f"{bad} elements within tolerance but not bit-exact"
    plan.destroy()
