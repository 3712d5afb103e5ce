"""Pins for the oracle's binary16 codec.

The pages fix fp16 parameters and gradients ("Where 16 bytes per parameter
comes from", state table, on the 16-byte-parameter page) and name its two
failure modes ("Why you can't just delete the fp32 copies": underflow below
2^-24, and swamping once the weight is about 2048x the update).  The oracle's
codec is its own bit-level code; here it is checked against numpy's binary16
cast (an independent round-to-nearest-even implementation) over every input,
and against what the IEEE format fixes.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest


def _nan_or_equal(ours, ref_bits):
    """Bit equality, except NaN outputs only need to be NaN of the same sign."""
    ref_nan = (ref_bits & 0x7C00) == 0x7C00
    ref_nan &= (ref_bits & 0x03FF) != 0
    our_nan = ((ours & 0x7C00) == 0x7C00) & ((ours & 0x03FF) != 0)
    same = ours == ref_bits
    ok = np.where(ref_nan, our_nan & ((ours >> 15) == (ref_bits >> 15)), same)
    return ok


def test_widen_every_fp16_pattern(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.array_equal(np.signbit(ours[nan]), np.signbit(ref[nan]))


_CHUNK = 1 << 24


def _narrow_chunk(start):
    import oracle
    x = np.arange(start, start + _CHUNK, dtype=np.uint32).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    ours = oracle.f32_to_f16(x)
    if np.array_equal(ours, ref):
        return []
    ok = _nan_or_equal(ours, ref)
    bad = np.flatnonzero(~ok)[:5]
    return [(int(x.view(np.uint32)[b]), int(ours[b]), int(ref[b])) for b in bad]


def test_narrow_every_fp32_pattern(orc):
    """All 2^32 binary32 bit patterns, against numpy's float32->float16."""
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ProcessPoolExecutor(workers) as ex:
        bad = [b for r in ex.map(_narrow_chunk, range(0, 1 << 32, _CHUNK)) for b in r]
    assert not bad, f"first mismatches (f32 bits, ours, numpy): {bad}"


def test_fp16_format_points(orc):
    """Points the binary16 format fixes: the smallest subnormal is 2^-24,
    the largest finite value 65504, 10 fraction bits (1 + 2^-10 is the next
    value after 1), and the round-to-nearest-even boundaries next to them."""
    c = orc.lib().orc_f32_to_f16
    w = orc.lib().orc_f16_to_f32
    assert c(2.0 ** -24) == 0x0001 and w(0x0001) == 2.0 ** -24
    assert c(2.0 ** -14) == 0x0400            # smallest normal
    assert w(0x7BFF) == 65504.0 and c(65504.0) == 0x7BFF
    assert c(65519.99) == 0x7BFF              # below the halfway point
    assert c(65520.0) == 0x7C00               # halfway ties to even -> inf
    assert c(1.0 + 2.0 ** -10) == 0x3C01
    assert c(1.0 + 2.0 ** -11) == 0x3C00      # tie -> even (1.0)
    assert c(1.0 + 3 * 2.0 ** -11) == 0x3C02  # tie -> even (1 + 2^-9)
    assert c(-0.0) == 0x8000 and c(0.0) == 0x0000
    assert c(float("inf")) == 0x7C00 and c(float("-inf")) == 0xFC00


def test_underflow_below_2_pow_minus_24(orc):
    """The page: magnitudes below 2^-24 cannot be held in fp16.  Under
    round-to-nearest-even the exact rule is: |x| <= 2^-25 becomes 0 (2^-25
    itself is a tie with the even neighbour 0), and (2^-25, 2^-24) rounds up
    to 2^-24.  Checked on every 61st binary32 value below 2^-24 and on every
    value within 2^16 patterns of 2^-25 (the full range is covered by the
    exhaustive comparison above)."""
    top = int(np.float32(2.0 ** -24).view(np.uint32))
    mid = int(np.float32(2.0 ** -25).view(np.uint32))
    lo = np.unique(np.concatenate([
        np.arange(0, top, 61, dtype=np.uint32),
        np.arange(mid - (1 << 16), mid + (1 << 16), dtype=np.uint32),
        np.arange(top - (1 << 16), top, dtype=np.uint32)]))
    x = lo.view(np.float32)
    h = orc.f32_to_f16(x)
    half = np.float32(2.0 ** -25)
    assert np.all(h[x <= half] == 0)
    assert np.all(h[x > half] == 1)
    assert np.all(orc.f32_to_f16(-x)[x <= half] == 0x8000)
    # a small learning rate (1e-3) times a small but representable fp16
    # gradient (2^-24 .. 2^-16) lands below 2^-25 and is lost in fp16
    g = orc.f16_to_f32(np.array([0x0001, 0x0010, 0x0100], np.uint16))
    step = (np.float32(1e-3) * g).astype(np.float32)
    assert np.all(orc.f32_to_f16(step) == 0)
    assert np.all(orc.f16_to_f32(np.array([0x0001, 0x0010, 0x0100], np.uint16)) > 0)


def _all_positive_finite_fp16():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    return bits, bits.view(np.float16).astype(np.float32)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_swamping_is_total_at_ratio_4096(orc, sign):
    """w + dw == w in fp16 for every positive finite fp16 w once
    |w| >= 4096 |dw|: |dw| is then at most half the spacing below and above w
    (a tie only at powers of two going down, which keeps the even w).  The
    sum w + w/4096 is exact in fp32 (11 + 12 significant bits), so one fp16
    rounding decides it."""
    bits, w = _all_positive_finite_fp16()
    dw = (w * np.float32(2.0 ** -12)).astype(np.float32)
    s = (w + np.float32(sign) * dw).astype(np.float32)
    assert np.array_equal(orc.f32_to_f16(s), bits)


def test_swamping_at_ratio_2048_only_at_ties(orc):
    """At exactly 2048x the page's rule is not yet total: +w/2048 is exactly
    half a spacing only when w is a power of two (a tie, kept at the even w),
    and it falls below half a spacing for subnormal w; every other w moves.
    Going down (-w/2048) only the subnormals and the smallest normal 2^-14
    (a tie toward the even 2^-14) keep w."""
    bits, w = _all_positive_finite_fp16()
    dw = (w * np.float32(2.0 ** -11)).astype(np.float32)
    up = orc.f32_to_f16((w + dw).astype(np.float32)) == bits
    down = orc.f32_to_f16((w - dw).astype(np.float32)) == bits
    subnormal = bits < 0x0400
    pow2 = (bits & 0x03FF) == 0
    assert np.array_equal(up, subnormal | pow2)
    assert np.array_equal(down, subnormal | (bits == 0x0400))
    assert up.sum() == 1023 + 30        # about 3.3% of 31,743 values
