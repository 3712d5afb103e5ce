"""GPU parity of the loss-scaled Adam step and the dynamic loss scale,
through the C ABI, against the oracle: every element and every field of
the scale's state compared after every step.  Each case prints its name
and sizes before it touches the GPU."""
import numpy as np
import pytest

import oracle
from parity import check16, check32, check_whole16, check_whole32, host16, host32, on_windows, to_dev32
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


def _half(fmt):
    import torch
    return torch.float16 if fmt == "f16" else torch.bfloat16


def _to_dev(bits, fmt):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(_half(fmt))


def _scaled_grads(n, seed, k, fmt):
    """N(0, 1e-3) gradients times 2^k, rounded to the format (bit patterns)."""
    g = np.random.default_rng(seed).standard_normal(n) * 1e-3 * 2.0 ** k
    if fmt == "f16":
        return g.astype(np.float16).view(np.uint16)
    return oracle.f32_to_bf16(g.astype(np.float32))


# (n, element offsets of param, grad, master, m, v): vector body, peeled
# head, single-element path, and tails
TENSORS = [(1, (0, 0, 0, 0, 0)), (4097, (0, 0, 0, 0, 0)), (70001, (3, 3, 3, 3, 3)),
           (5000, (1, 0, 0, 0, 0)), (1 << 16, (0, 0, 0, 0, 0))]


def _plan(zs, fmt, seed):
    import torch
    rng = np.random.default_rng(seed)
    dev, host = [], []
    for n, offs in TENSORS:
        bufs = [torch.zeros(n + o + 8, dtype=dt, device="cuda")[o:o + n]
                for o, dt in zip(offs, (_half(fmt), _half(fmt), torch.float32, torch.float32,
                                        torch.float32))]
        w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        bufs[2].copy_(to_dev32(w0))
        dev.append(bufs)
        host.append([np.zeros(n, np.uint16), w0.copy(), np.zeros(n, np.float32),
                     np.zeros(n, np.float32)])
    create = zs.zero_plan_create
    plan = create([tuple(b) for b in dev])
    return plan, dev, host


def _compare(dev, host, fmt, what):
    bad = 0
    for (p, g, w, m, v), (hp_, hw, hm, hv) in zip(dev, host):
        bad += check16(host16(p), hp_, what + " param", fmt=fmt)["not_bit_exact"]
        bad += check32(host32(w), hw, what + " master")["not_bit_exact"]
        bad += check32(host32(m), hm, what + " m")["not_bit_exact"]
        bad += check32(host32(v), hv, what + " v")["not_bit_exact"]
    return bad


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("k", [0, 8, 24, -3, 100, 150])
def test_scaled_step_matches_oracle(zs, fmt, k):
    """Three scaled steps over five tensors (every access path); k = 150 is
    stored in the state and clamped to 100 by the step."""
    import torch
    say(f"scaled step fmt={fmt} k={k}")
    plan, dev, host = _plan(zs, fmt, 7 + k)
    ls = zs.LossScale(log2_scale=0, device=torch.device("cuda", 0))
    ls.state[0] = k
    k_eff = max(-100, min(100, k))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t in range(1, 4):
        for j, ((p, g, w, m, v), h) in enumerate(zip(dev, host)):
            # the gradients' own factor stays where the format holds them
            gb = _scaled_grads(g.numel(), 100 * t + j, min(k_eff, 12 if fmt == "f16" else 30),
                               fmt)
            g.copy_(_to_dev(gb, fmt))
            assert oracle.adam_step_scaled(gb, h[0], h[1], h[2], h[3], t=t, log2_scale=k_eff,
                                           fmt=fmt, **HP) == 0
        zs.zero_adam_step(plan, zs.AdamHParams(**HP), t, flag, loss_scale=ls)
        torch.cuda.synchronize()
        assert _compare(dev, host, fmt, f"{fmt} k={k} t={t}") == 0
    assert int(flag.item()) == 0
    assert ls.read() == (k, 0, 0, 0)            # the step never writes the scale
    plan.destroy()


@pytest.mark.parametrize("k", [-1, 0])
def test_bf16_overflow_after_unscale_raises_the_flag(zs, k):
    """bfloat16 gradients of the largest finite magnitude, at scattered
    positions over every access path: at k = -1 their product with 2^-k is
    infinite in fp32, which the flag reports (and master, m, v go NaN as in
    the oracle); at k = 0 they stay finite and the flag stays down."""
    import torch
    say(f"bf16 overflow after unscale k={k}")
    plan, dev, host = _plan(zs, "bf16", 31 - k)
    ls = zs.LossScale(log2_scale=0, min_log2=-100, device=torch.device("cuda", 0))
    ls.state[0] = k
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    want = 0
    for j, ((p, g, w, m, v), h) in enumerate(zip(dev, host)):
        gb = _scaled_grads(g.numel(), 500 + j, 0, "bf16")
        pos = np.unique(np.random.default_rng(j).integers(0, g.numel(), 3))
        gb[pos] = np.where(pos % 2 == 0, 0x7F7F, 0xFF7F).astype(np.uint16)
        g.copy_(_to_dev(gb, "bf16"))
        want |= oracle.adam_step_scaled(gb, h[0], h[1], h[2], h[3], t=1, log2_scale=k,
                                        fmt="bf16", **HP)
    assert want == (1 if k < 0 else 0)
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1, flag, loss_scale=ls)
    torch.cuda.synchronize()
    assert _compare(dev, host, "bf16", f"bf16 overflow k={k}") == 0
    assert int(flag.item()) == want
    plan.destroy()


def test_update_matches_oracle(zs):
    """A fixed sequence of flags written from the host; after each update
    the device state equals the oracle's and the flag is 0 again."""
    import torch
    say("loss scale update sequence")
    rng = np.random.default_rng(11)
    flags = (rng.random(300) < 0.2).astype(int)
    flags[:40] = 0
    for interval, lo, hi, k0 in ((3, 0, 6, 2), (1, -4, 4, 0), (7, 10, 10, 10), (2, -100, 100, 99)):
        ls = zs.LossScale(log2_scale=k0, interval=interval, min_log2=lo, max_log2=hi)
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        st = (k0, 0, 0, 0)
        for f in flags:
            flag.fill_(int(f) * 5)             # any nonzero value is an overflow
            ls.update(flag)
            st = oracle.loss_scale_update(st, int(f), interval=interval, min_log2=lo,
                                          max_log2=hi)
            torch.cuda.synchronize()
            assert ls.read() == st
            assert int(flag.item()) == 0


def test_reduce_scaled_step_update_loop(zs):
    """The whole chain over 12 steps, N_d = 4 fp16 slices: reduce (flag) ->
    scaled step skipped on the flag -> scale update (clears the flag).
    Slices carry the current scale; at steps 3, 7 and 8 one slice holds an
    infinity, so those steps are skipped, the scale halves and t does not
    advance.  Arrays and scale state equal the oracle's after every step."""
    import torch
    nd, n = 4, 9001
    say(f"reduce -> scaled step -> update, nd={nd} n={n}")
    rng = np.random.default_rng(12)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p = torch.zeros(n, dtype=torch.float16, device="cuda")
    g = torch.zeros(n, dtype=torch.float16, device="cuda")
    w, m, v = to_dev32(w0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    plan = zs.zero_plan_create([(p, g, w, m, v)])
    ls = zs.LossScale(log2_scale=12, interval=2, min_log2=0, max_log2=14)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp_, hw, hm, hv = np.zeros(n, np.uint16), w0.copy(), np.zeros(n, np.float32), \
        np.zeros(n, np.float32)
    st = (12, 0, 0, 0)
    t = 1
    for step in range(1, 13):
        k = st[0]
        hs = [_scaled_grads(n, 1000 * step + r, k, "f16") for r in range(nd)]
        if step in (3, 7, 8):
            hs[step % nd][(step * 977) % n] = 0x7C00
        ds = [_to_dev(h, "f16") for h in hs]
        zs.zero_reduce_grad_shard(ds, g, flag)
        zs.zero_adam_step(plan, zs.AdamHParams(**HP), t, skip_if_nonzero=flag, loss_scale=ls)
        ls.update(flag)
        ref, rflag = oracle.reduce_grad(hs)
        assert rflag == int(step in (3, 7, 8))
        oracle.adam_step_scaled(ref, hp_, hw, hm, hv, t=t, log2_scale=k, skip=bool(rflag), **HP)
        st = oracle.loss_scale_update(st, rflag, interval=2, min_log2=0, max_log2=14)
        torch.cuda.synchronize()
        assert ls.read() == st
        assert int(flag.item()) == 0
        bad = (check16(host16(p), hp_, f"loop {step} param")["not_bit_exact"]
               + check32(host32(w), hw, f"loop {step} master")["not_bit_exact"]
               + check32(host32(m), hm, f"loop {step} m")["not_bit_exact"]
               + check32(host32(v), hv, f"loop {step} v")["not_bit_exact"])
        assert bad == 0
        t += 0 if rflag else 1
    assert st[2] == 3 and st[3] == 9
    plan.destroy()


def test_scaled_rejects(zs):
    import torch
    say("scaled step argument checks")
    n = 64
    p = torch.zeros(n, dtype=torch.float16, device="cuda")
    g = torch.zeros(n, dtype=torch.float16, device="cuda")
    w, m, v = (torch.zeros(n, device="cuda") for _ in range(3))
    plan = zs.zero_plan_create([(p, g, w, m, v)])
    ls = zs.LossScale()
    with pytest.raises(zs.ZeroError):           # the flag inside the scale record
        zs.zero_adam_step(plan, zs.AdamHParams(**HP), 1, ls.state[1:2], loss_scale=ls)
    with pytest.raises(zs.ZeroError):
        ls.update(ls.state[2:3])
    with pytest.raises(ValueError):
        zs.LossScale(min_log2=5, max_log2=4)
    with pytest.raises(ValueError):
        zs.LossScale(interval=0)
    plan.destroy()


def test_flat_7p5b_nd64_loss_scaled_full_size(zs):
    """The launch configuration bench.py times with --loss-scale 16, at full
    size: rank 0's 117,187,500-element partition of Psi = 7.5e9 over 64
    ranks, two steps of reduce of the 64 fp16 slices -> Adam on gradients
    read as carrying 2^16 (skipped on the reduce's flag) -> the scale's
    update (interval 2000, 2^0..2^24).  Every element equals the oracle's,
    recomputed from the same slices (threaded over windows); the scale's
    state is (16, 2, 0, 2) after the two finite steps."""
    import torch
    wl = W.WORKLOADS["flat_7p5b_nd64"]
    lay = zs.zero_shard_layout(wl.psi, wl.nd, wl.rank, wl.align)
    n = lay.real_len
    say(f"loss-scaled flat_7p5b_nd64 n={n}")
    full, sh = W.device_flat_state(wl, lay.offset, n, lay.padded_total)
    buf, rows = W.device_slices(wl, n)
    plan = zs.zero_plan_create([sh.arrays()])
    ls = zs.LossScale(log2_scale=16, interval=2000, min_log2=0, max_log2=24)
    w0 = host32(sh.w)
    slices = [host16(r) for r in rows]
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t in (1, 2):
        zs.zero_reduce_grad_shard(rows, sh.g, flag)
        zs.zero_adam_step(plan, zs.AdamHParams(**HP), t, skip_if_nonzero=flag, loss_scale=ls)
        ls.update(flag)
    torch.cuda.synchronize()
    assert ls.read() == (16, 2, 0, 2) and int(flag.item()) == 0
    got = [host16(sh.p), host32(sh.w), host32(sh.m), host32(sh.v)]
    say("loss-scaled flat_7p5b_nd64: oracle over the whole shard")
    g_ref = np.empty(n, np.uint16)
    rflag = on_windows(lambda lo, hi: oracle.reduce_grad([x[lo:hi] for x in slices],
                                                         g_ref[lo:hi])[1], n)
    assert rflag == 0
    del slices
    rp, rw = np.zeros(n, np.uint16), w0
    rm, rv = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in (1, 2):
        on_windows(lambda lo, hi: oracle.adam_step_scaled(g_ref[lo:hi], rp[lo:hi], rw[lo:hi],
                                                          rm[lo:hi], rv[lo:hi], t=t,
                                                          log2_scale=16, **HP), n)
    res = [check_whole16(got[0], rp, "loss-scaled nd64 param"),
           check_whole32(got[1], rw, "loss-scaled nd64 master"),
           check_whole32(got[2], rm, "loss-scaled nd64 m"),
           check_whole32(got[3], rv, "loss-scaled nd64 v")]
    say(f"loss-scaled full size: all {n} elements, not bit-exact {[r['not_bit_exact'] for r in res]}")
    assert sum(r["not_bit_exact"] for r in res) == 0
    plan.destroy()
    del full, sh, buf, rows
