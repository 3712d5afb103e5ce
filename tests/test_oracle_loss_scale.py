"""Pins for the oracle's loss-scaled Adam step and its dynamic loss scale.

The pages do not treat loss scaling.  They do say why fp16 gradients need
help: values below 2^-24 are lost in fp16 ("Why you can't just delete the
fp32 copies" on the 16-byte-parameter page).  The reading built here: the
gradients carry a factor 2^k; the step multiplies each widened gradient by
2^-k before the unscaled update; a step whose gradients hold a non-finite
value is skipped and the scale halves; a run of finite steps doubles it.

What pins it, without re-typing the oracle:
  * k = 0 is the unscaled step, bit for bit;
  * multiplying by a power of two is exact, so on gradients whose scaled
    value is still an fp16 (or bfloat16) number the scaled step equals the
    unscaled step on the true gradient, bit for bit, over several steps;
  * gradients too small for fp16 (2^-30 scale) are lost without a scale
    (the pages' underflow) and recovered with k = 24, against the fp64 closed
    form of the first Adam step;
  * the scale's state machine against a sequence traced by hand, and its
    invariants over random flag sequences.
"""
import numpy as np
import pytest

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _state(n, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    return w, np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)


def _bits(x, fmt):
    x = np.asarray(x, np.float64)
    if fmt == "f16":
        h = x.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), x), "value not exact in fp16"
        return h.view(np.uint16)
    f = x.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), x)
    u = f.view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "value not exact in bfloat16"
    return (u >> 16).astype(np.uint16)


def _true_grads(n, seed, lo_exp, hi_exp, fmt):
    """Gradients that are exact fp16 (or bfloat16) numbers: a random sign, a
    random 10-bit (7-bit) fraction, exponents in [lo_exp, hi_exp)."""
    rng = np.random.default_rng(seed)
    frac_bits = 10 if fmt == "f16" else 7
    frac = 1.0 + rng.integers(0, 1 << frac_bits, n) / float(1 << frac_bits)
    e = rng.integers(lo_exp, hi_exp, n)
    s = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return s * np.ldexp(frac, e)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_zero_scale_is_the_plain_step(orc, fmt):
    n = 3000
    a, b = _state(n, 1), _state(n, 1)
    for t in range(1, 4):
        g = _bits(_true_grads(n, 10 + t, -12, 2, fmt), fmt)
        fa = orc.adam_step(g, a[3], a[0], a[1], a[2], t=t, fmt=fmt, **HP)
        fb = orc.adam_step_scaled(g, b[3], b[0], b[1], b[2], t=t, log2_scale=0, fmt=fmt, **HP)
        assert fa == fb == 0
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32 if x.dtype == np.float32 else np.uint16),
                              y.view(np.uint32 if y.dtype == np.float32 else np.uint16))


@pytest.mark.parametrize("fmt,k", [("f16", 1), ("f16", 8), ("f16", 14), ("f16", -4),
                                   ("bf16", 8), ("bf16", 40), ("bf16", -30)])
def test_power_of_two_scale_is_exact(orc, fmt, k):
    """Four steps on scaled gradients 2^k g (exact in the format) with
    log2_scale = k equal four unscaled steps on g, every bit of every array."""
    n = 4000
    a, b = _state(n, 2), _state(n, 2)
    for t in range(1, 5):
        g = _true_grads(n, 20 + t, -10, 0, fmt)
        fa = orc.adam_step(_bits(g, fmt), a[3], a[0], a[1], a[2], t=t, fmt=fmt, **HP)
        fb = orc.adam_step_scaled(_bits(np.ldexp(g, k), fmt), b[3], b[0], b[1], b[2], t=t,
                                  log2_scale=k, fmt=fmt, **HP)
        assert fa == fb == 0
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32 if x.dtype == np.float32 else np.uint16),
                              y.view(np.uint32 if y.dtype == np.float32 else np.uint16))
    # and the scale is not a no-op: the same scaled gradients read unscaled
    # give a different state
    c = _state(n, 2)
    g = _true_grads(n, 21, -10, 0, fmt)
    orc.adam_step(_bits(np.ldexp(g, k), fmt), c[3], c[0], c[1], c[2], t=1, fmt=fmt, **HP)
    assert not np.array_equal(c[1], a[1])


def test_scale_recovers_gradients_below_fp16(orc):
    """True gradients of magnitude 2^-30..2^-29 round to zero in fp16, so an
    unscaled step does not move the master at all (the pages' underflow);
    with a scale of 2^24 they arrive as fp16 normals, and one step from
    m = v = 0 gives m = (1-b1) g, v = (1-b2) g^2 and w1 = w0 - lr g/(|g|+eps)
    (bias corrections cancel at t = 1), each within 1e-6 relative of fp64
    (w0 in [0.5, 1), so that w1 stays far from zero)."""
    n = 5000
    g = _true_grads(n, 30, -30, -29, "f16")
    assert np.all(np.abs(g) < 2.0 ** -25)
    lost = g.astype(np.float16)
    assert np.all(lost == 0)
    w, m, v, p = _state(n, 3)
    w0 = w.copy()
    orc.adam_step(lost.view(np.uint16), p, w, m, v, t=1, **HP)
    assert np.array_equal(w, w0) and np.all(m == 0) and np.all(v == 0)

    w, m, v, p = _state(n, 3)
    w[:] = 0.5 + 0.5 * np.random.default_rng(31).random(n)    # far from zero
    w0 = w.copy()
    flag = orc.adam_step_scaled(_bits(np.ldexp(g, 24), "f16"), p, w, m, v, t=1, log2_scale=24,
                                **HP)
    assert flag == 0
    b1, b2, lr, eps = HP["beta1"], HP["beta2"], HP["lr"], HP["eps"]

    def rel(got, ex):
        return float(np.max(np.abs(got.astype(np.float64) - ex) / np.abs(ex)))

    assert rel(m, (1 - b1) * g) <= 1e-6
    assert rel(v, (1 - b2) * g * g) <= 1e-6
    step_ex = lr * g / (np.abs(g) + eps)
    assert float(np.max(np.abs((w0.astype(np.float64) - w) - step_ex) / np.abs(step_ex))) <= 1e-3
    assert rel(w, w0.astype(np.float64) - step_ex) <= 1e-6


def test_scaled_flag_skip_and_range(orc):
    from oracle import OracleError
    n = 64
    g = _bits(_true_grads(n, 40, -8, 0, "f16"), "f16")
    g[17] = 0x7C00
    w, m, v, p = _state(n, 4)
    assert orc.adam_step_scaled(g, p, w, m, v, t=1, log2_scale=5, **HP) == 1
    assert np.isnan(w[17]) and np.isfinite(np.delete(w, 17)).all()
    w, m, v, p = _state(n, 4)
    w0 = w.copy()
    assert orc.adam_step_scaled(g, p, w, m, v, t=1, log2_scale=5, skip=True, **HP) == 0
    assert np.array_equal(w, w0) and np.all(m == 0) and np.all(p == 0)
    for k in (-101, 101):
        with pytest.raises(OracleError):
            orc.adam_step_scaled(g, p, w, m, v, t=1, log2_scale=k, **HP)


def test_scaled_flag_sees_the_unscaled_gradient(orc):
    """The flag tests the gradient the update uses, after 2^-k.  bfloat16
    has the fp32 exponent range, so its largest finite value (2^127 (2 -
    2^-7)) times 2^1 (k = -1) is infinite in fp32: the flag is raised and,
    per IEEE arithmetic, the master becomes NaN (inf / inf in the update).
    At k = 0 the same value is finite: no flag, and since g * g overflows,
    v is infinite and the update's denominator with it, so the master does
    not move.  fp16's largest value times 2^100 is about 6.6e34, finite:
    no fp16 gradient raises the flag at any |k| <= 100."""
    big = np.ldexp(2.0 - 2.0 ** -7, 127)
    g = _bits([big, -big, 1.0], "bf16")
    w, m, v, p = _state(3, 9)
    w0 = w.copy()
    assert orc.adam_step_scaled(g, p, w, m, v, t=1, log2_scale=-1, fmt="bf16", **HP) == 1
    assert np.isnan(w[:2]).all() and np.isfinite(w[2])
    w, m, v, p = w0.copy(), np.zeros(3, np.float32), np.zeros(3, np.float32), p * 0
    assert orc.adam_step_scaled(g, p, w, m, v, t=1, log2_scale=0, fmt="bf16", **HP) == 0
    assert np.isinf(v[:2]).all() and np.array_equal(w[:2], w0[:2])
    g16 = _bits([65504.0, -65504.0, 2.0 ** -24], "f16")
    for k in (-100, -1, 0, 100):
        w, m, v, p = _state(3, 9)
        assert orc.adam_step_scaled(g16, p, w, m, v, t=1, log2_scale=k, **HP) == 0, k


def test_loss_scale_sequence_traced_by_hand(orc):
    """interval 3, scale exponents in [0, 4], starting at 2^2."""
    flags = [0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 1, 1, 1, 1, 0, 0, 0, 0]
    want = [(2, 1, 0, 1), (2, 2, 0, 2), (3, 0, 0, 3),     # third finite step: double
            (3, 1, 0, 4), (3, 2, 0, 5), (4, 0, 0, 6),
            (4, 1, 0, 7), (4, 2, 0, 8), (4, 0, 0, 9),     # capped at 2^4, count restarts
            (3, 0, 1, 9),                                 # overflow: halve, skip
            (3, 1, 1, 10),
            (2, 0, 2, 10), (1, 0, 3, 10), (0, 0, 4, 10),
            (0, 0, 5, 10),                                # floored at 2^0
            (0, 1, 5, 11), (0, 2, 5, 12), (1, 0, 5, 13), (1, 1, 5, 14)]
    st = (2, 0, 0, 0)
    for f, w in zip(flags, want):
        st = orc.loss_scale_update(st, f, interval=3, min_log2=0, max_log2=4)
        assert st == w


def test_loss_scale_invariants(orc):
    rng = np.random.default_rng(5)
    for trial in range(200):
        interval = int(rng.integers(1, 7))
        lo = int(rng.integers(-5, 5))
        hi = lo + int(rng.integers(0, 8))
        k0 = int(rng.integers(lo, hi + 1))
        p_bad = rng.random() * 0.5
        st = (k0, 0, 0, 0)
        run = 0
        for s in range(1, 60):
            f = int(rng.random() < p_bad)
            prev = st
            st = orc.loss_scale_update(st, f, interval=interval, min_log2=lo, max_log2=hi)
            assert lo <= st[0] <= hi and 0 <= st[1] < interval
            assert st[2] + st[3] == s
            run = 0 if f else run + 1
            assert st[1] == run % interval
            assert abs(st[0] - prev[0]) <= 1
        # all finite from a fresh state: k grows by one every interval steps
        st = (lo, 0, 0, 0)
        for s in range(1, 40):
            st = orc.loss_scale_update(st, 0, interval=interval, min_log2=lo, max_log2=hi)
            assert st[0] == min(hi, lo + s // interval)
