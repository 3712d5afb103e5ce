"""Pins for the oracle's gradient reduction over N_d fp16 slices.

After the reduce-scatter each rank owns the final gradients of its partition
("The part that sounds too good: communication" on the 16-byte-parameter page;
the communication paragraph of "The Mathematics" on the ZeRO and the Memory
Tricks page).  The oracle averages the N_d fp16 slices with an fp32 sum in
rank order and rounds the mean to fp16.  Expected values here come from exact
arithmetic: fp16 values are integer multiples of 2^-24 below 2^16, so a sum of
up to 2^13 of them is exact in float64.
"""
import math

import numpy as np
import pytest

U = 2.0 ** -24


def _rand_slices(rng, nd, n, std=1e-3):
    return [(rng.standard_normal(n) * std).astype(np.float16) for _ in range(nd)]


def _ulp16(x):
    x = np.abs(np.asarray(x, np.float64)).astype(np.float16)
    nxt = np.nextafter(x, np.float16(np.inf))
    return (nxt.astype(np.float64) - x.astype(np.float64))


@pytest.mark.parametrize("nd", [1, 2, 3, 4, 8, 64, 256])
def test_identical_slices_reduce_to_themselves(orc, nd):
    """The mean of N_d copies of x is x bit for bit: every partial sum j*x is
    exact in fp32 (11 + 13 bits) and (N_d x) / N_d = x."""
    rng = np.random.default_rng(nd)
    bits = rng.integers(0, 0x7C00, 4096, dtype=np.uint16) | (
        rng.integers(0, 2, 4096, dtype=np.uint16) << 15)
    out, flag = orc.reduce_grad([bits] * nd)
    assert flag == 0
    # -0 stays -0 only when every term is -0 (fp32 -0 + -0 = -0)
    assert np.array_equal(out, bits)


def test_single_slice_is_a_bit_copy(orc):
    """N_d = 1 is a copy of every fp16 pattern (NaNs stay NaN, signs kept)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    out, flag = orc.reduce_grad([bits])
    nan = ((bits & 0x7C00) == 0x7C00) & ((bits & 0x3FF) != 0)
    assert np.array_equal(out[~nan], bits[~nan])
    assert np.all(((out[nan] & 0x7C00) == 0x7C00) & ((out[nan] & 0x3FF) != 0))
    assert flag == 1


@pytest.mark.parametrize("nd", [2, 3, 4, 7, 8, 64])
def test_mean_within_summation_bound(orc, nd):
    """|out - exact_mean| <= (N_d - 1) u sum|x_r| / N_d (recursive fp32
    summation) + u |mean| (the division) + half an fp16 ulp of the result.
    Where the sum carries no rounding (all |terms| and partial sums are
    multiples of the final quantum) the result is the nearest fp16 exactly."""
    rng = np.random.default_rng(100 + nd)
    n = 20000
    sl = _rand_slices(rng, nd, n)
    out, flag = orc.reduce_grad(sl)
    assert flag == 0
    x = np.stack([s.astype(np.float64) for s in sl])
    exact = x.sum(axis=0) / nd            # exact sum (multiples of 2^-24)
    absum = np.abs(x).sum(axis=0)
    got = out.view(np.float16).astype(np.float64)
    bound = (nd - 1) * U * absum / nd + U * np.abs(exact) + 0.5 * _ulp16(got) + 1e-300
    assert np.all(np.abs(got - exact) <= bound * (1 + 1e-12))
    nearest = exact.astype(np.float16).astype(np.float64)   # numpy RNE of exact
    assert (got == nearest).mean() > 0.999


def test_exact_integer_means(orc):
    """Small integers sum exactly in fp32, so the output is the fp16 nearest
    to the exact mean, including ties (resolved to even)."""
    rng = np.random.default_rng(3)
    for nd in (2, 4, 5, 8, 64):
        sl = [rng.integers(-1000, 1000, 5000).astype(np.float16) for _ in range(nd)]
        out, _ = orc.reduce_grad(sl)
        exact = np.stack([s.astype(np.float64) for s in sl]).sum(0) / nd
        assert np.array_equal(out, exact.astype(np.float16).view(np.uint16))


def test_rank_order_summation(orc):
    """fp32 addition is not associative; the oracle sums in rank order from
    slice 0.  With a = 2^11, b = -2^11, c = 2^-14 (all fp16): in order
    (a + b) + c = 2^-14, while summing from the last slice, c + b is a tie
    halfway between two fp32 values next to -2^11 that rounds to the even
    -2^11, and c is lost.  Mean over 3."""
    a, b, c = np.float16(2048.0), np.float16(-2048.0), np.float16(2.0 ** -14)
    out, _ = orc.reduce_grad([np.array([a]), np.array([b]), np.array([c])])
    want = np.float32(np.float32(2.0 ** -14) / np.float32(3))
    assert out.view(np.float16)[0] == np.float16(want) != 0
    assert np.float32(np.float32(c) + np.float32(b)) == np.float32(b)
    # 1 + 2^-24 + ... : slice 0 = 1, the others each add 2^-24; in fp32 each
    # 1 + 2^-24 ties back to 1, so the rank-order sum stays 1
    nd = 5
    sl = [np.array([np.float16(1.0)])] + [np.array([np.float16(2.0 ** -24)])] * (nd - 1)
    out, _ = orc.reduce_grad(sl)
    assert out.view(np.float16)[0] == np.float16(np.float32(1.0) / np.float32(nd))


def test_non_finite_outputs_raise_the_flag(orc):
    """+inf and -inf in one column give NaN; an overflowing sum of finite
    values gives inf only if the mean itself overflows fp16 (the fp32 sum
    does not overflow), so 4 x 65504 averages back to 65504."""
    ok = np.array([1.0, 2.0, 3.0], np.float16)
    pinf = np.array([np.inf, 2.0, 3.0], np.float16)
    ninf = np.array([-np.inf, 2.0, 3.0], np.float16)
    out, flag = orc.reduce_grad([pinf, ninf, ok])
    assert flag == 1 and np.isnan(out.view(np.float16)[0])
    assert np.array_equal(out[1:].view(np.float16), np.array([2.0, 3.0], np.float16))
    big = np.array([65504.0], np.float16)
    out, flag = orc.reduce_grad([big] * 4)
    assert flag == 0 and out.view(np.float16)[0] == np.float16(65504.0)
    out, flag = orc.reduce_grad([np.array([np.inf], np.float16), big])
    assert flag == 1 and out.view(np.float16)[0] == np.inf
    out, flag = orc.reduce_grad([ok, ok])
    assert flag == 0
    nan = np.array([np.nan, 1.0, 2.0], np.float16)
    out, flag = orc.reduce_grad([nan, ok])
    assert flag == 1 and np.isnan(out.view(np.float16)[0])


def test_empty_and_rejects(orc):
    out, flag = orc.reduce_grad([np.zeros(0, np.float16)] * 4)
    assert out.size == 0 and flag == 0
    with pytest.raises(orc.OracleError):
        orc.reduce_grad([])
