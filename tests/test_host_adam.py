"""The host CPU Adam step (zero_adam_step_host: the update ZeRO-Offload runs
on the CPU) against the oracle, on the CPU: every fp16 and every bfloat16
gradient pattern, ragged sizes split over several thread counts, unaligned
arrays, the narrowing of millions of master bit patterns in both formats,
the non-finite flag and the argument checks.  Bit-exact is the bar, as for the
GPU kernel: both do the same IEEE binary32 operations in the same order."""
import numpy as np
import pytest

from parity import check16, check32

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


@pytest.fixture(scope="module")
def zs():
    from zero_partitioned_mixed_layout_amd import build, zero_shard
    if build.stale():
        pytest.fail("libzeroshard.so is older than its sources: run __graft_entry__.build()")
    return zero_shard


def _state(rng, n, warm):
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32) if warm else np.zeros(n, np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32) if warm else np.zeros(n, np.float32)
    return w, m, v


def _both(zs, orc, g, w, m, v, t, threads=0):
    n = g.size
    p, P = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    W, M, V = w.copy(), m.copy(), v.copy()
    flag = np.zeros(1, np.int32)
    zs.zero_adam_step_host(g, p, w, m, v, zs.AdamHParams(**HP), t, threads=threads,
                           nonfinite_flag=flag)
    rflag = orc.adam_step(g, P, W, M, V, t=t, **HP)
    return (p, w, m, v, int(flag[0])), (P, W, M, V, rflag)


def _exact(got, ref, what):
    p, w, m, v, f = got
    P, W, M, V, F = ref
    res = [check16(p, P, what + " param"), check32(w, W, what + " master"),
           check32(m, M, what + " m"), check32(v, V, what + " v")]
    assert f == F
    assert sum(r["not_bit_exact"] for r in res) == 0, what


def test_every_fp16_gradient_pattern(zs, orc):
    n = 1 << 16
    g = np.arange(n, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(1)
    for t, warm in ((1, False), (9, True)):
        w, m, v = _state(rng, n, warm)
        got, ref = _both(zs, orc, g, w, m, v, t)
        _exact(got, ref, f"all patterns t={t}")
        assert got[4] == 1


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_ragged_sizes(zs, orc, threads):
    rng = np.random.default_rng(threads)
    for n in (1, 7, 8, 9, 15, 16, 17, 1000, 70001):
        for t, warm in ((1, False), (7, True)):
            g = (rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
            w, m, v = _state(rng, n, warm)
            got, ref = _both(zs, orc, g, w, m, v, t, threads)
            _exact(got, ref, f"n={n} threads={threads} t={t}")
            assert got[4] == 0


def test_unaligned_arrays(zs, orc):
    """Arrays one element past a 32-byte boundary (the vector loads are
    unaligned loads)."""
    rng = np.random.default_rng(5)
    n = 4099
    g = np.zeros(n + 1, np.uint16)[1:]
    g[:] = (rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
    w, m, v = (np.zeros(n + 1, np.float32)[1:] for _ in range(3))
    w0, m0, v0 = _state(rng, n, True)
    w[:], m[:], v[:] = w0, m0, v0
    p = np.zeros(n + 1, np.uint16)[1:]
    W, M, V, P = w0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)
    zs.zero_adam_step_host(g, p, w, m, v, zs.AdamHParams(**HP), 2)
    orc.adam_step(np.ascontiguousarray(g), P, W, M, V, t=2, **HP)
    assert np.array_equal(p, P)
    for a, b in ((w, W), (m, M), (v, V)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_flag_and_ieee_propagation(zs, orc):
    rng = np.random.default_rng(9)
    n = 1000
    g = (rng.standard_normal(n) * 1e-3).astype(np.float16).view(np.uint16)
    g[[3, 500, 999]] = [0x7C00, 0xFC00, 0x7E00]
    w, m, v = _state(rng, n, True)
    got, ref = _both(zs, orc, g, w, m, v, 3, threads=4)
    _exact(got, ref, "injected inf/nan")
    assert got[4] == 1


def test_rejects(zs):
    n = 64
    g, p = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    w, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    hp = zs.AdamHParams(**HP)
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_adam_step_host(g, p, w, m, m, hp, 1)           # m is v
    assert e.value.status == -1
    with pytest.raises(zs.ZeroError):
        zs.zero_adam_step_host(g, p, w, m, v, hp, 0)           # t = 0
    with pytest.raises(zs.ZeroError):
        zs.zero_adam_step_host(g, p, w, m, v, zs.AdamHParams(weight_decay=0.1), 1)
    raw = np.zeros(4 * n + 4, np.uint8)
    w_odd = raw[1:1 + 4 * n].view(np.float32)                  # not 4-byte aligned
    with pytest.raises(zs.ZeroError):
        zs.zero_adam_step_host(g, p, w_odd, m, v, hp, 1)
    with pytest.raises(ValueError):
        zs.zero_adam_step_host(g[:10], p, w, m, v, hp, 1)
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_adam_step_host(g, p, w, m, v, hp, 1, threads=1025)   # above the bound
    assert e.value.status == -1
    zs.zero_adam_step_host(g, p, w, m, v, hp, 1, threads=1024)       # at the bound
    # n = 0 does nothing
    e16, e32 = np.zeros(0, np.uint16), np.zeros(0, np.float32)
    zs.zero_adam_step_host(e16, e16.copy(), e32, e32.copy(), e32.copy(), hp, 1)


def _both_fmt(zs, orc, g, w, m, v, t, fmt, threads=0):
    n = g.size
    p, P = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    W, M, V = w.copy(), m.copy(), v.copy()
    flag = np.zeros(1, np.int32)
    zs.zero_adam_step_host(g, p, w, m, v, zs.AdamHParams(**HP), t, threads=threads,
                           nonfinite_flag=flag, fmt=fmt)
    rflag = orc.adam_step(g, P, W, M, V, t=t, fmt=fmt, **HP)
    return (p, w, m, v, int(flag[0])), (P, W, M, V, rflag)


def _exact_fmt(got, ref, what, fmt):
    p, w, m, v, f = got
    P, W, M, V, F = ref
    res = [check16(p, P, what + " param", fmt=fmt), check32(w, W, what + " master"),
           check32(m, M, what + " m"), check32(v, V, what + " v")]
    assert f == F
    assert sum(r["not_bit_exact"] for r in res) == 0, what


def test_bf16_every_gradient_pattern(zs, orc):
    n = 1 << 16
    g = np.arange(n, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(11)
    for t, warm in ((1, False), (9, True)):
        w, m, v = _state(rng, n, warm)
        got, ref = _both_fmt(zs, orc, g, w, m, v, t, "bf16")
        _exact_fmt(got, ref, f"bf16 all patterns t={t}", "bf16")
        assert got[4] == 1


@pytest.mark.parametrize("threads", [1, 3])
def test_bf16_ragged_sizes(zs, orc, threads):
    rng = np.random.default_rng(20 + threads)
    for n in (1, 7, 8, 9, 17, 1000, 70001):
        for t, warm in ((1, False), (7, True)):
            g = orc.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
            w, m, v = _state(rng, n, warm)
            got, ref = _both_fmt(zs, orc, g, w, m, v, t, "bf16", threads)
            _exact_fmt(got, ref, f"bf16 n={n} threads={threads} t={t}", "bf16")
            assert got[4] == 0


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_narrowing_of_master_bit_patterns(zs, orc, fmt):
    """With g = 0 and m = v = 0 the step leaves every master unchanged (its
    update is 0 / eps = 0), so the written parameter is the narrowing of the
    master itself: 4 Mi random fp32 bit patterns (every class: zeros,
    subnormals, normals, values that round to infinity, infinities, NaNs)
    plus the halfway cases of the target format, through both the
    eight-wide and the single-element code, against the oracle's narrowing
    (NaN compared by class)."""
    rng = np.random.default_rng(31 if fmt == "f16" else 32)
    bits = rng.integers(0, 1 << 32, size=(1 << 22) + 5, dtype=np.uint64).astype(np.uint32)
    if fmt == "bf16":
        ties = (rng.integers(0, 1 << 16, size=4096, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    else:
        # fp32 values exactly halfway between two fp16 neighbours (13 low bits 0x1000)
        ties = (rng.integers(0x33000, 0x47800, size=4096, dtype=np.uint64).astype(np.uint32) << 13) | 0x1000
    bits[:4096] = ties
    w = bits.view(np.float32).copy()
    n = w.size
    g = np.zeros(n, np.uint16)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    p = np.zeros(n, np.uint16)
    zs.zero_adam_step_host(g, p, w, m, v, zs.AdamHParams(**HP), 1, fmt=fmt)
    want = orc.f32_to_bf16(bits.view(np.float32)) if fmt == "bf16" else orc.f32_to_f16(bits.view(np.float32))
    # the master is unchanged, except that IEEE arithmetic quiets a signaling NaN
    nan = np.isnan(bits.view(np.float32))
    assert np.array_equal(w.view(np.uint32)[~nan], bits[~nan]) and np.isnan(w[nan]).all()
    assert check16(p, want, f"{fmt} narrowing", fmt=fmt)["not_bit_exact"] == 0
