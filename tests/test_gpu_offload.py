"""GPU parity of the ZeRO-Offload step (zero_offload_step): fp16 gradients
to the host, the CPU update over host fp32 state, fp16 parameters back.
Against the oracle on small and ragged shards, with pipeline chunks small
enough that every staging slot is reused many times; and against the GPU
Adam kernel, bit for bit over the whole arrays, on the 7.5e9 / N_d = 64
rank's 117,187,500-element shard.  Each case prints its name and sizes before
it touches the GPU."""
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


@pytest.mark.parametrize("chunk,threads", [(64, 1), (4096, 4), (0, 0)])
def test_offload_matches_oracle(zs, chunk, threads):
    import torch
    off = zs.zero_offload_create(chunk, threads)
    rng = np.random.default_rng(chunk + threads)
    for n in (1, 7, 63, 64, 65, 200, 4095, 4097, 70001):
        say(f"offload chunk={chunk} threads={threads} n={n}")
        g = (rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
        if n > 100:
            g[[5, n // 2]] = [0x7C00, 0xFE00]          # an inf and a NaN
        w = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = (rng.random(n) * 1e-6).astype(np.float32)
        W_, M_, V_, P_ = w.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
        dg = to_dev16(g)
        dp = torch.zeros(n, dtype=torch.float16, device="cuda")
        flag = np.zeros(1, np.int32)
        off.step(dg, dp, w, m, v, zs.AdamHParams(**HP), 5, nonfinite_flag=flag)
        rflag = oracle.adam_step(g, P_, W_, M_, V_, t=5, **HP)
        res = [check16(host16(dp), P_, "param"), check32(w, W_, "master"),
               check32(m, M_, "m"), check32(v, V_, "v")]
        assert sum(r["not_bit_exact"] for r in res) == 0
        assert int(flag[0]) == rflag == (1 if n > 100 else 0)
    off.destroy()


def test_offload_steps_chain(zs):
    """Three steps in a row on one pipeline equal three oracle steps."""
    import torch
    n = 10_007
    off = zs.zero_offload_create(1024, 3)
    rng = np.random.default_rng(17)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    W_, M_, V_, P_ = w.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
    dp = torch.zeros(n, dtype=torch.float16, device="cuda")
    for t in (1, 2, 3):
        say(f"offload chain t={t}")
        g = (rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
        off.step(to_dev16(g), dp, w, m, v, zs.AdamHParams(**HP), t)
        oracle.adam_step(g, P_, W_, M_, V_, t=t, **HP)
        assert np.array_equal(host16(dp), P_)
    for a, b in ((w, W_), (m, M_), (v, V_)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    off.destroy()


def test_offload_rejects(zs):
    import torch
    say("offload rejects")
    off = zs.zero_offload_create(1024, 2)
    n = 256
    g = torch.zeros(n, dtype=torch.float16, device="cuda")
    p = torch.zeros(n, dtype=torch.float16, device="cuda")
    w, m, v = (np.zeros(n, np.float32) for _ in range(3))
    hp = zs.AdamHParams(**HP)
    with pytest.raises(zs.ZeroError):
        off.step(g, g, w, m, v, hp, 1)             # param is the gradient
    with pytest.raises(zs.ZeroError):
        off.step(g, p, w, m, m, hp, 1)             # m is v
    with pytest.raises(zs.ZeroError):
        off.step(g, p, w, m, v, hp, 0)             # t = 0
    with pytest.raises(ValueError):
        off.step(g[:10], p, w, m, v, hp, 1)
    with pytest.raises(zs.ZeroError):
        zs.zero_offload_create(1001, 1)            # chunk not a multiple of 8
    off.destroy()


def test_offload_equals_gpu_step_at_full_size(zs):
    """The 117,187,500-element shard (Psi = 7.5e9, N_d = 64, rank 0): the
    offload step against zero_adam_step on a copy of the same state, every
    element of every array bit for bit."""
    import time
    import torch
    wl = W.WORKLOADS["flat_7p5b_nd64"]
    lay = zs.zero_shard_layout(wl.psi, wl.nd, 0, wl.align)
    n = lay.real_len
    say(f"offload full size n={n}")
    t_ = W.DeviceTensor(n, "cuda")
    W.device_normal(n, W.MASTER_STD, W.master_seed(wl.seed), None, "cuda", out=t_.w)
    W.device_fill_grads(wl, [t_], 1)
    w, m, v = host32(t_.w).copy(), host32(t_.m).copy(), host32(t_.v).copy()
    dp = torch.zeros(n, dtype=torch.float16, device="cuda")
    off = zs.zero_offload_create()
    hp = zs.AdamHParams(**HP)
    t0 = time.perf_counter()
    off.step(t_.g, dp, w, m, v, hp, 1)
    dt = time.perf_counter() - t0
    plan = zs.zero_plan_create([t_.arrays()])
    zs.zero_adam_step(plan, hp, 1)
    torch.cuda.synchronize()
    say(f"offload step {dt * 1e3:.1f} ms ({n / dt / 1e9:.2f} G params/s)")
    assert torch.equal(dp.view(torch.int16), t_.p.view(torch.int16))
    for a, d in ((w, t_.w), (m, t_.m), (v, t_.v)):
        assert np.array_equal(a.view(np.uint32), host32(d).view(np.uint32))
    plan.destroy()
    off.destroy()
    del t_, dp, w, m, v
    gc.collect()
    torch.cuda.empty_cache()


def _to_devbf(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("chunk,threads", [(64, 1), (0, 0)])
def test_offload_bf16_matches_oracle(zs, chunk, threads):
    """The bfloat16 offload step (zero_offload_step_bf16): bfloat16 gradient
    and parameter on the device, the host update over fp32 state, against
    the oracle's bfloat16 step, with an infinity and a NaN injected."""
    import torch
    off = zs.zero_offload_create(chunk, threads)
    rng = np.random.default_rng(300 + chunk + threads)
    for n in (1, 7, 65, 4097, 70001):
        say(f"offload bf16 chunk={chunk} threads={threads} n={n}")
        g = oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
        if n > 100:
            g[[5, n // 2]] = [0x7F80, 0xFFC0]          # an inf and a NaN
        w = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = (rng.random(n) * 1e-6).astype(np.float32)
        W_, M_, V_, P_ = w.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
        dp = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        flag = np.zeros(1, np.int32)
        off.step(_to_devbf(g), dp, w, m, v, zs.AdamHParams(**HP), 4, nonfinite_flag=flag)
        rflag = oracle.adam_step(g, P_, W_, M_, V_, t=4, fmt="bf16", **HP)
        res = [check16(host16(dp), P_, "param", fmt="bf16"), check32(w, W_, "master"),
               check32(m, M_, "m"), check32(v, V_, "v")]
        assert sum(r["not_bit_exact"] for r in res) == 0
        assert int(flag[0]) == rflag == (1 if n > 100 else 0)
    off.destroy()


def test_offload_describe(zs):
    """zero_offload_describe: the thread count asked for (or the default,
    at most 16 and at most the CPUs available), the chunk, and a NUMA
    placement consistent with the host's sysfs: pinned CPUs only where the
    GPU's node is known, never more than the process may use."""
    import os
    say("offload describe")
    cpus = len(os.sched_getaffinity(0))
    off = zs.zero_offload_create(2048, 3)
    i = off.info()
    assert i["threads"] == 3 and i["chunk_elems"] == 2048
    assert i["numa_node"] >= -1
    assert 0 <= i["pinned_cpus"] <= cpus
    if i["numa_node"] == -1:
        assert i["pinned_cpus"] == 0
    off.destroy()
    off = zs.zero_offload_create()
    d = off.info()
    assert d["chunk_elems"] == 4 << 20
    assert 1 <= d["threads"] <= min(16, cpus)
    assert d["numa_node"] == i["numa_node"]
    off.destroy()
    with pytest.raises(ValueError):
        off.info()
