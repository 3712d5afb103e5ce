"""zero_adam_step_noalloc against zero_adam_step (through a plan) on the GPU.

The allocation-free entry point rebuilds the chunk table in the library's
fixed per-device array at every call; its results must be bit-identical to
the plan path's on the same inputs.  Each test makes two calls in a row, the
second over a smaller input, so the second call runs on an array that still
holds the first call's (larger) table."""
import numpy as np
import pytest
import torch

from zero_partitioned_mixed_layout_amd import workloads as W

pytestmark = pytest.mark.gpu

HP = dict(W.ADAM_HP)


@pytest.fixture(scope="module")
def zs():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from zero_partitioned_mixed_layout_amd import zero_shard
    return zero_shard


def _bits(x):
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32).cpu().numpy()


class State:
    """Five flat buffers and a list of tensor views into them; `shift`
    puts the parameter views one element off the other arrays' phase from
    tensor `shift_from` on (single-element path)."""

    def __init__(self, sizes, seed, shift_from=None):
        dev = torch.device("cuda")
        total = sum(sizes) + 8 * len(sizes) + 64
        r = np.random.Generator(np.random.Philox(seed))
        self.p = torch.zeros(total, dtype=torch.float16, device=dev)
        self.g = torch.from_numpy((r.standard_normal(total) * 1e-3).astype(np.float16)).to(dev)
        self.w = torch.from_numpy((r.standard_normal(total) * 0.02).astype(np.float32)).to(dev)
        self.m = torch.from_numpy((r.standard_normal(total) * 1e-4).astype(np.float32)).to(dev)
        self.v = torch.from_numpy((r.random(total) * 1e-6).astype(np.float32)).to(dev)
        self.views = []
        off = 0
        for k, n in enumerate(sizes):
            po = off + (1 if shift_from is not None and k >= shift_from else 0)
            self.views.append((self.p[po:po + n], self.g[off:off + n], self.w[off:off + n],
                               self.m[off:off + n], self.v[off:off + n]))
            off += n + 8

    def clone(self):
        c = State.__new__(State)
        c.p, c.g, c.w, c.m, c.v = (x.clone() for x in (self.p, self.g, self.w, self.m, self.v))
        c.views = []
        for vs in self.views:
            c.views.append(tuple(
                getattr(c, nm)[x.storage_offset():x.storage_offset() + x.numel()]
                for nm, x in zip("pgwmv", vs)))
        return c

    def arrays(self):
        return [_bits(x) for x in (self.p, self.g, self.w, self.m, self.v)]


def _same(a, b, what):
    for nm, x, y in zip("pgwmv", a.arrays(), b.arrays()):
        bad = np.flatnonzero(x != y)
        assert bad.size == 0, f"{what}: {nm} differs at {bad.size} elements, first {bad[:5]}"


def _step_both(zs, A, B, idx, t, flagged=False):
    """One step over the tensors idx: A through zero_adam_step_noalloc, B
    through a plan and zero_adam_step; returns both flags."""
    fa = torch.zeros(1, dtype=torch.int32, device="cuda")
    fb = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step_noalloc([A.views[k] for k in idx], zs.AdamHParams(**HP), t, fa)
    plan = zs.zero_plan_create([B.views[k] for k in idx])
    zs.zero_adam_step(plan, zs.AdamHParams(**HP), t, fb)
    torch.cuda.synchronize()
    plan.destroy()
    return int(fa.item()), int(fb.item())


def test_noalloc_matches_plan_two_calls_second_smaller(zs):
    sizes = [1, 3, 513, 16384 + 7, 100_000, 1_000_003, 4_194_304 + 5]
    print(f"noalloc: tensors {sizes}", flush=True)
    A = State(sizes, seed=11)
    B = A.clone()
    fa, fb = _step_both(zs, A, B, range(len(sizes)), t=3)
    _same(A, B, "first call (7 tensors, 5.3M elements)")
    assert fa == fb == 0
    # the second call: fewer, smaller tensors (the array still holds the
    # first call's longer table)
    fa, fb = _step_both(zs, A, B, [1, 2, 4], t=4)
    _same(A, B, "second call (3 tensors, 100,516 elements)")
    assert fa == fb == 0


def test_noalloc_many_tensors_single_path_and_flag(zs):
    # 100 tensors (four staging launches of at most 32), the last 40 with the
    # parameter one element off (single elements), one infinite gradient
    rs = np.random.Generator(np.random.Philox(5))
    sizes = [int(x) for x in rs.integers(1, 70_000, size=100)]
    print(f"noalloc: 100 tensors, {sum(sizes)} elements", flush=True)
    A = State(sizes, seed=12, shift_from=60)
    A.views[70][1][min(5, sizes[70] - 1)] = float("inf")
    B = A.clone()
    fa, fb = _step_both(zs, A, B, range(100), t=7)
    _same(A, B, "first call (100 tensors)")
    assert fa == fb == 1
    fa, fb = _step_both(zs, A, B, [0, 61], t=8)
    _same(A, B, "second call (2 tensors)")
    assert fa == fb == 0


def test_noalloc_skip_leaves_everything(zs):
    A = State([4099, 77], seed=13)
    before = A.arrays()
    skip = torch.ones(1, dtype=torch.int32, device="cuda")
    zs.zero_adam_step_noalloc(A.views, zs.AdamHParams(**HP), 1, None, skip)
    torch.cuda.synchronize()
    for nm, x, y in zip("pgwmv", before, A.arrays()):
        assert np.array_equal(x, y), nm
    # and a smaller call after it still matches the plan path
    B = A.clone()
    fa, fb = _step_both(zs, A, B, [1], t=2)
    _same(A, B, "call after a skipped one")


def test_noalloc_limit_is_checked_before_launch(zs):
    """More tensors than the array holds descriptors for are refused
    (ERANGE) before anything is enqueued; a call after it works."""
    A = State([1000, 2000], seed=14)
    before = A.arrays()
    too_many = [A.views[0]] * (zs.ZERO_NOALLOC_MAX_TENSORS + 1)
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_adam_step_noalloc(too_many, zs.AdamHParams(**HP), 1)
    assert e.value.status == zs.ZERO_ERANGE
    torch.cuda.synchronize()
    for nm, x, y in zip("pgwmv", before, A.arrays()):
        assert np.array_equal(x, y), nm
    B = A.clone()
    fa, fb = _step_both(zs, A, B, [0, 1], t=1)
    _same(A, B, "call after a refused one")
