"""Pins for the oracle's bfloat16 variant of the step.

[DSZ] "Why parameter count is not training memory" notes that BF16 setups
differ in which states they keep; this variant keeps the 16-byte ledger
with bfloat16 parameters and gradients in place of fp16.  The oracle's
bfloat16 codec (its own quantum arithmetic) is checked against torch's CPU
bfloat16 cast (an independent round-to-nearest-even implementation) on
every binary32 input, widening against the format's definition (the
binary32 with the same top 16 bits), and the bfloat16 Adam and reduce
against the already-pinned fp16 ones on values both formats hold exactly.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
_CHUNK = 1 << 24


def _narrow_chunk(start):
    import torch
    import oracle
    x = np.arange(start, start + _CHUNK, dtype=np.uint32).view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.f32_to_bf16(x)
    if np.array_equal(ours, ref):
        return []
    nan_ref = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    nan_our = ((ours & 0x7F80) == 0x7F80) & ((ours & 0x7F) != 0)
    # a NaN in gives a NaN out; its sign and payload are not fixed by the
    # format (torch's vectorised cast returns 0xFFFF, the oracle 0x7FC0 with
    # the input's sign), and the comparison rules compare NaN by class only
    ok = np.where(nan_ref, nan_our, ours == ref)
    bad = np.flatnonzero(~ok)[:5]
    return [(int(x.view(np.uint32)[b]), int(ours[b]), int(ref[b])) for b in bad]


def test_narrow_every_fp32_pattern(orc):
    """All 2^32 binary32 bit patterns, against torch's float32->bfloat16
    (NaN by class)."""
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ProcessPoolExecutor(workers) as ex:
        bad = [b for r in ex.map(_narrow_chunk, range(0, 1 << 32, _CHUNK)) for b in r]
    assert not bad, f"first mismatches (f32 bits, ours, torch): {bad}"


def test_widen_every_bf16_pattern(orc):
    bits = np.arange(1 << 16, dtype=np.uint32)
    ours = orc.bf16_to_f32(bits.astype(np.uint16))
    ref = (bits << 16).astype(np.uint32).view(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_format_points(orc):
    c, w = orc.lib().orc_f32_to_bf16, orc.lib().orc_bf16_to_f32
    assert c(1.0) == 0x3F80 and c(1.0 + 2.0 ** -7) == 0x3F81
    assert c(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even (1.0)
    assert c(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (1 + 2^-6)
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127         # largest finite
    assert w(0x7F7F) == big and c(big) == 0x7F7F
    assert c(float("inf")) == 0x7F80 and c(float("-inf")) == 0xFF80
    assert w(0x0001) == 2.0 ** -133              # smallest subnormal
    assert c(-0.0) == 0x8000 and c(0.0) == 0x0000
    # the overflow boundary: the halfway point to 2^128 ties to the even 2^128
    halfway = np.array([0x7F7F8000, 0x7F7F7FFF], np.uint32).view(np.float32)
    assert c(float(halfway[0])) == 0x7F80 and c(float(halfway[1])) == 0x7F7F


def _both_formats(rng, n):
    """Gradients that fp16 and bfloat16 both hold exactly: at most 8
    significant bits, magnitudes in fp16's normal range (or zero)."""
    k = rng.integers(-255, 256, n).astype(np.float64)
    e = rng.integers(-22, -8, n)
    x = (k * np.exp2(e)).astype(np.float32)
    x[np.abs(x) < 2.0 ** -14] = 0.0
    g16 = orc_module().f32_to_f16(x)
    gbf = orc_module().f32_to_bf16(x)
    assert np.array_equal(orc_module().f16_to_f32(g16), x)
    assert np.array_equal(orc_module().bf16_to_f32(gbf), x)
    return g16, gbf


def orc_module():
    import oracle
    return oracle


@pytest.mark.parametrize("t", [1, 6])
def test_bf16_adam_state_equals_fp16_adam_state(orc, t):
    """On gradients both formats hold exactly, the fp32 master, m and v of
    the bfloat16 step equal those of the fp16 step bit for bit, and each
    16-bit parameter is its format's rounding of the same master."""
    rng = np.random.default_rng(t)
    n = 50_000
    g16, gbf = _both_formats(rng, n)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32) if t > 1 else np.zeros(n, np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32) if t > 1 else np.zeros(n, np.float32)
    a = [w.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)]
    b = [w.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)]
    fa = orc.adam_step(g16, a[3], a[0], a[1], a[2], t=t, **HP)
    fb = orc.adam_step(gbf, b[3], b[0], b[1], b[2], t=t, fmt="bf16", **HP)
    assert fa == fb == 0
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(a[3], orc.f32_to_f16(a[0]))
    assert np.array_equal(b[3], orc.f32_to_bf16(b[0]))


def test_bf16_adam_non_finite(orc):
    """bfloat16 infinities and NaNs raise the flag and propagate per IEEE
    exactly as the fp16 ones of the same value do."""
    n = 6
    gbf = np.array([0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0x0000, 0x8000], np.uint16)
    g16 = np.array([0x7C00, 0xFC00, 0x7E00, 0x3C00, 0x0000, 0x8000], np.uint16)
    w = np.linspace(-1, 1, n).astype(np.float32)
    a = [w.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)]
    b = [w.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)]
    assert orc.adam_step(g16, a[3], a[0], a[1], a[2], t=1, **HP) == 1
    assert orc.adam_step(gbf, b[3], b[0], b[1], b[2], t=1, fmt="bf16", **HP) == 1
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(np.isnan(x), np.isnan(y))
        fin = ~np.isnan(x)
        assert np.array_equal(x[fin].view(np.uint32), y[fin].view(np.uint32))


def test_bf16_reduce(orc):
    """Identical slices reduce to themselves; one slice is a bit copy of all
    65,536 patterns (NaN class kept); integer means that bfloat16 holds come
    out exactly; the fp32 sum runs in rank order (1, 2^25, -2^25 gives 0,
    the reverse order would give 1/3)."""
    rng = np.random.default_rng(2)
    x = orc.f32_to_bf16((rng.standard_normal(10_000) * 1e-3).astype(np.float32))
    for nd in (1, 2, 7, 64):
        out, f = orc.reduce_grad([x] * nd, fmt="bf16")
        assert np.array_equal(out, x) and f == 0
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    out, f = orc.reduce_grad([bits], fmt="bf16")
    nan = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)
    assert f == 1
    assert np.array_equal(out[~nan], bits[~nan])
    assert np.all(((out[nan] & 0x7F80) == 0x7F80) & ((out[nan] & 0x7F) != 0))
    for nd in (2, 4, 8):
        k = rng.integers(-16, 17, (nd, 5000))
        vals = (k * 2.0 ** -10).astype(np.float32)
        sl = [orc.f32_to_bf16(v) for v in vals]
        out, f = orc.reduce_grad(sl, fmt="bf16")
        exact = (k.sum(axis=0) * 2.0 ** -10 / nd).astype(np.float32)
        # nd in {2, 4, 8}: the mean has at most 7 significant bits
        assert np.array_equal(out, orc.f32_to_bf16(exact)) and f == 0
    order = [orc.f32_to_bf16(np.array([v], np.float32)) for v in (1.0, 2.0 ** 25, -(2.0 ** 25))]
    out, _ = orc.reduce_grad(order, fmt="bf16")
    assert out[0] == 0x0000
    out, _ = orc.reduce_grad(order[::-1], fmt="bf16")
    assert orc.bf16_to_f32(out)[0] == orc.bf16_to_f32(orc.f32_to_bf16(np.array([1 / 3], np.float32)))[0]
    # the flag: values of the largest finite exponent leave it down, an
    # infinite mean raises it, and so does a sum that leaves the fp32 range
    # (twice the largest finite bfloat16 is past fp32's largest number)
    big = np.array([0x7F7F, 0xFF7F, 0x7F00, 0x0001], np.uint16)
    out, f = orc.reduce_grad([big], fmt="bf16")
    assert f == 0 and np.array_equal(out, big)
    out, f = orc.reduce_grad([np.array([0x3F80, 0x7F80], np.uint16)], fmt="bf16")
    assert f == 1 and out[1] == 0x7F80
    out, f = orc.reduce_grad([np.array([0x7F7F], np.uint16)] * 2, fmt="bf16")
    assert f == 1 and out[0] == 0x7F80


def test_bf16_swamping_is_worse_than_fp16(orc):
    """bfloat16 keeps 8 significant bits: an update smaller than the weight
    by 2^9 (512x, not fp16's 2048x) is lost by a naive bf16 update for every
    positive finite weight whose update is itself a normal bf16 number
    (w >= 2^-117; below that the update's own rounding in the subnormal
    range can grow it to half an ulp of w), which is why the fp32 master is
    kept."""
    w_bits = np.arange(0x0500, 0x7F80, dtype=np.uint16)      # 2^-117 <= w, finite
    w = orc.bf16_to_f32(w_bits).astype(np.float64)
    dw = w / 512.0
    upd = orc.f32_to_bf16((w + orc.bf16_to_f32(orc.f32_to_bf16(dw.astype(np.float32)))).astype(np.float32))
    assert np.all(upd == w_bits)
