"""The C ABI without a GPU: the library loads, exports every function the
header declares, and its host-only functions (layout, ledger, step scalars,
plan classification, argument checks) agree with the oracle and the header.
No call here reaches a device: the checks that hand fake device addresses to
entry points which launch once their arguments pass run in a child process
that sees no GPU, so a check that regressed fails with EHIP instead of
launching a kernel on made-up memory."""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

from zero_partitioned_mixed_layout_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_shard.h")


@pytest.fixture(scope="module")
def zs():
    from zero_partitioned_mixed_layout_amd import build, zero_shard
    if build.stale():
        pytest.fail("libzeroshard.so is older than its sources: run __graft_entry__.build()")
    return zero_shard


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(zs):
    names = _declared()
    assert len(names) >= 10
    missing = [n for n in names if not hasattr(zs.lib(), n)]
    assert not missing
    assert sorted(zs.EXPORTS) == names


def _without_devices(body: str) -> None:
    """Run the module-level function `body`(zs) in a child process in which
    HIP sees no device."""
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="",
               ROCR_VISIBLE_DEVICES="")
    here = os.path.dirname(os.path.abspath(__file__))
    code = (f"import sys; sys.path[:0] = [{ROOT!r}, {here!r}]; import test_abi_host as t; "
            f"from zero_partitioned_mixed_layout_amd import zero_shard as zs; "
            f"t.{body}(zs); print('BODY_OK')")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "BODY_OK" in r.stdout, r.stdout + r.stderr


def test_status_strings(zs):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert zs.zero_status_str(code) != "unknown status"
    assert zs.zero_status_str(7) == "unknown status"


def test_layout_matches_oracle(zs, orc):
    for psi in list(range(0, 130)) + [2 ** 20, 7_500_000_000, 2 ** 63 + 5]:
        for nd in (1, 2, 3, 4, 7, 8, 64):
            for align in (1, 2, 8, 512):
                for rank in sorted({0, 1 % nd, nd // 2, nd - 1}):
                    try:
                        want = orc.shard_layout(psi, nd, rank, align)
                    except orc.OracleError:
                        with pytest.raises(zs.ZeroError):
                            zs.zero_shard_layout(psi, nd, rank, align)
                        continue
                    assert zs.zero_shard_layout(psi, nd, rank, align)._asdict() == want


def test_layout_rejects(zs):
    for args, code in (((10, 0, 0, 1), -1), ((10, 4, 4, 1), -1), ((10, 4, 0, 0), -1),
                       ((2 ** 64 - 1, 3, 0, 512), -2)):
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_shard_layout(*args)
        assert e.value.status == code
    assert zs.lib().zero_shard_layout(1, 1, 0, 1, None) == -1


def test_ledger_matches_oracle(zs, orc):
    for psi in (0, 1, 99, 2 ** 20, 1_557_611_200, 6_738_415_616, 7_500_000_000, 2 ** 59):
        for nd in (1, 3, 8, 64, 1000):
            for align in (1, 512):
                for stage in range(4):
                    want = orc.state_bytes(stage, psi, nd, align)
                    assert zs.zero_state_bytes(stage, psi, nd, align) == want
    with pytest.raises(zs.ZeroError):
        zs.zero_state_bytes(4, 10, 1)
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_state_bytes(0, 2 ** 61, 1)
    assert e.value.status == -2


def test_ledger_workload_check(zs):
    """ZeRO-2 on one rank of Psi = 7.5e9 over 64 ranks: fp16 params for all
    Psi, the rank's fp16 gradient shard and its fp32 master, m and v."""
    psi, nd = 7_500_000_000, 64
    S = zs.zero_shard_layout(psi, nd, 0).shard_len
    assert zs.zero_state_bytes(2, psi, nd) == 2 * psi + 2 * S + 3 * 4 * S == 16_640_625_000


@pytest.mark.parametrize("b1,b2", [(0.9, 0.999), (0.8, 0.95), (0.0, 0.5)])
def test_scalars_match_oracle_bit_for_bit(zs, orc, b1, b2):
    for t in list(range(1, 300)) + [4096, 10 ** 6, 2 ** 40]:
        for lr, eps in ((1e-3, 1e-8), (0.1, 0.0), (3e-4, 1e-6)):
            got = np.array(zs.zero_adam_scalars(zs.AdamHParams(lr, b1, b2, eps), t), np.float32)
            want = orc.adam_scalars(lr, b1, b2, eps, t)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (t, lr, eps)


def test_scalars_reject(zs):
    H = zs.AdamHParams
    for hp, t in ((H(), 0), (H(weight_decay=0.01), 1), (H(beta1=1.0), 1), (H(beta2=-0.1), 1),
                  (H(eps=-1e-8), 1), (H(lr=float("nan")), 1), (H(eps=float("inf")), 1)):
        with pytest.raises(zs.ZeroError):
            zs.zero_adam_scalars(hp, t)


def _fake(n, p=0x100000, g=0x200000, w=0x300000, m=0x400000, v=0x500000):
    return (p, g, w, m, v, n)


def test_plan_describe_paths(zs):
    # all five arrays aligned: everything on the four-element vector path
    d = zs.zero_plan_describe([_fake(100)])
    assert (d["vector_elems"], d["scalar_elems"]) == (100, 0)
    d = zs.zero_plan_describe([_fake(103)])
    assert (d["vector_elems"], d["scalar_elems"]) == (100, 3)
    # all five arrays two elements past an aligned boundary: peel 2 singly,
    # then vectors, then the last 2 singly
    d = zs.zero_plan_describe([_fake(100, 0x100004, 0x200004, 0x300008, 0x400008, 0x500008)])
    assert (d["vector_elems"], d["scalar_elems"]) == (96, 4)
    # fp16 arrays 8-byte aligned but not 16: still the vector path
    d = zs.zero_plan_describe([_fake(100, 0x100008, 0x200008)])
    assert (d["vector_elems"], d["scalar_elems"]) == (100, 0)
    # fp16 param one element off the grad's phase: single elements below
    # 1,024 elements; from 1,024 the other arrays stay on the vector path
    # (the parameter's stores shifted), for every phase of the parameter
    d = zs.zero_plan_describe([_fake(100, 0x100002)])
    assert (d["vector_elems"], d["scalar_elems"]) == (0, 100)
    d = zs.zero_plan_describe([_fake(1023, 0x100002)])
    assert (d["vector_elems"], d["scalar_elems"]) == (0, 1023)
    for p in (0x100002, 0x100004, 0x100006, 0x100102):
        d = zs.zero_plan_describe([_fake(1024, p)])
        assert (d["vector_elems"], d["scalar_elems"]) == (1024, 0), hex(p)
        d = zs.zero_plan_describe([_fake(1027, p)])
        assert (d["vector_elems"], d["scalar_elems"]) == (1024, 3), hex(p)
    # the state two elements past 1 KiB: a head of 254 (2 singly), the
    # parameter off by one more element
    d = zs.zero_plan_describe([_fake(1030, 0x100006, 0x200004, 0x300008, 0x400008, 0x500008)])
    assert (d["vector_elems"], d["scalar_elems"]) == (1028, 2)
    # the gradient off instead, or both 16-bit arrays: the vector path from
    # 1,024 elements (the gradient's loads shifted too), single below
    for g, p in (((1 << 41) + 2, 1 << 40), ((1 << 41) + 6, (1 << 40) + 2)):
        d = zs.zero_plan_describe([_fake(1 << 20, p, g, 1 << 42, 1 << 43, 1 << 44)])
        assert (d["vector_elems"], d["scalar_elems"]) == (1 << 20, 0)
        d = zs.zero_plan_describe([_fake(1000, p, g, 1 << 42, 1 << 43, 1 << 44)])
        assert (d["vector_elems"], d["scalar_elems"]) == (0, 1000)
    # the fp32 arrays disagreeing: single elements at any size
    d = zs.zero_plan_describe([_fake(1 << 20, 1 << 40, 1 << 41, 1 << 42, (1 << 43) + 4,
                                     1 << 44)])
    assert (d["vector_elems"], d["scalar_elems"]) == (0, 1 << 20)
    # fp32 master one element off: single elements
    d = zs.zero_plan_describe([_fake(100, w=0x300004)])
    assert (d["vector_elems"], d["scalar_elems"]) == (0, 100)


def test_plan_chunking(zs):
    """Chunk counts: a tensor's first chunk holds its peeled head plus up to
    chunk_elems elements, then chunk_elems each."""
    d = zs.zero_plan_describe([_fake(1 << 20, 1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44)])
    assert d["chunk_elems"] == 16384 and d["n_chunks"] == 64
    d = zs.zero_plan_describe([_fake(40000)])            # 16384 would leave 17 of 96 slots idle
    assert d["chunk_elems"] == 8192 and d["n_chunks"] == 5
    for C in (512, 1024, 4096, 1 << 24):
        for n in (1, 511, 512, 513, 5000, 100003):
            d = zs.zero_plan_describe([_fake(n)], C)
            assert d["chunk_elems"] == C and d["n_chunks"] == -(-n // C), (C, n)
    # fp32 arrays 8 bytes past a 1 KiB boundary: from 1,024 elements the
    # head runs to the element where they reach the next one (254 = 2
    # singly, then 63 fours), riding in the first chunk: 254 + 512, then 512
    two = (0x100004, 0x200004, 0x300008, 0x400008, 0x500008)
    assert zs.zero_plan_describe([_fake(254 + 1024, *two)], 512)["n_chunks"] == 2
    assert zs.zero_plan_describe([_fake(254 + 1025, *two)], 512)["n_chunks"] == 3
    # below 1,024 elements the head stays at the vector's 2
    assert zs.zero_plan_describe([_fake(2 + 512, *two)], 512)["n_chunks"] == 1
    assert zs.zero_plan_describe([_fake(2 + 513, *two)], 512)["n_chunks"] == 2
    assert zs.zero_plan_describe([_fake(1023, *two)], 512)["n_chunks"] == 2
    # the same vector head of 2, but v reaches its 1 KiB boundary 4
    # elements earlier than master and m: the head stays at the vector's 2
    off_v = (0x100004, 0x200004, 0x300008, 0x400008, 0x500018)
    assert zs.zero_plan_describe([_fake(2 + 1024, *off_v)], 512)["n_chunks"] == 2
    assert zs.zero_plan_describe([_fake(2 + 1025, *off_v)], 512)["n_chunks"] == 3
    for C in (1, 100, 511, 513, 1000, (1 << 24) + 512, 2 ** 31):
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_plan_describe([_fake(10)], C)
        assert e.value.status == -1


def _slots_and_work(sizes, C, tile=512):
    """Tile slots (chunks x 512-element tiles per chunk) and tiles holding
    work, for aligned tensors (no head), counted tile by tile."""
    slots = work = 0
    for n in sizes:
        chunks = max(1, -(-n // C))
        slots += chunks * (C // tile)
        for c in range(chunks):
            cnt = min(C, n - c * C)
            work += max(1, -(-cnt // tile))
    return slots, work


def test_plan_chunk_choice(zs):
    """With chunk_elems = 0 the plan takes the largest of 16384 ... 512 whose
    workgroup slots exceed the tiles with work by at most one eighth: model
    lists and big shards keep 16384, many small tensors get small chunks,
    and an explicit chunk size is kept as given."""
    rng = np.random.default_rng(12)
    cases = [[1 << 26], [1024] * 100000, list(rng.integers(1, 601, 4000)),
             [50_000_000] + [4096] * 10000, list(rng.integers(1, 100_000, 300)),
             [n for _, n in W.WORKLOADS["llama_7b"].tensors],
             [n for _, n in W.WORKLOADS["gpt2_xl"].tensors]]
    for sizes in cases:
        ents, base = [], 1 << 40
        for n in sizes:
            n = int(n)
            step = (n * 4 + 1023) // 1024 * 1024   # every array on 1 KiB: no head
            ents.append(_fake(n, base, base + step, base + 2 * step, base + 3 * step,
                              base + 4 * step))
            base += 5 * step
        C = zs.zero_plan_describe(ents)["chunk_elems"]
        want = 512
        for c in (16384, 8192, 4096, 2048, 1024):
            sl, wk = _slots_and_work([int(n) for n in sizes], c)
            if sl <= wk + wk // 8:
                want = c
                break
        assert C == want, (len(sizes), C, want)
    assert zs.zero_plan_describe([_fake(1024)] * 1)["chunk_elems"] == 1024
    big = [_fake(1024, (1 << 40) + k * (1 << 20), (1 << 41) + k * (1 << 20), (1 << 42) + k * (1 << 20),
                 (1 << 43) + k * (1 << 20), (1 << 44) + k * (1 << 20)) for k in range(1000)]
    assert zs.zero_plan_describe(big)["chunk_elems"] == 1024
    assert zs.zero_plan_describe(big, 16384)["chunk_elems"] == 16384


def test_plan_tile_choice(zs):
    """The step's tile: 256 elements per wave when at least 7/8 of the
    plan's elements take the vector path and the chunk is 16384 (big
    tensors), else 512."""
    def tile(ents, chunk=0):
        return zs.zero_plan_describe(ents, chunk)["tile_elems"]
    big = _fake(1 << 26, 1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44)
    assert tile([big]) == 256
    assert tile([big], 16384) == 256
    assert tile([big], 8192) == 512                       # not the default chunk
    single = _fake(1 << 26, 1 << 40, 1 << 41, (1 << 42) + 4, 1 << 43, 1 << 44)
    assert zs.zero_plan_describe([single])["scalar_elems"] == 1 << 26
    assert tile([single]) == 512                           # all single elements
    small = [_fake(1024, (1 << 40) + k * (1 << 20), (1 << 41) + k * (1 << 20),
                   (1 << 42) + k * (1 << 20), (1 << 43) + k * (1 << 20),
                   (1 << 44) + k * (1 << 20)) for k in range(1000)]
    assert tile(small) == 512                              # the plan takes 1024-element chunks
    # exactly 1/8 of the elements single: still 256; a little more: 512
    vec = _fake(7 << 20, 1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44)
    for n_single, want in ((1 << 20, 256), ((1 << 20) + 8, 512)):
        one = _fake(n_single, 1 << 45, 3 << 44, (1 << 46) + 4, 5 << 44, 7 << 44)
        d = zs.zero_plan_describe([vec, one])
        assert d["scalar_elems"] == n_single and d["tile_elems"] == want, (n_single, d)
    for name in ("llama_7b", "gpt2_xl"):
        ents, base = [], 1 << 40
        for _, n in W.WORKLOADS[name].tensors:
            step = (n * 4 + 1023) // 1024 * 1024   # every array on 1 KiB: no head
            ents.append(_fake(n, base, base + step, base + 2 * step, base + 3 * step, base + 4 * step))
            base += 5 * step
        assert tile(ents) == 256, name


def test_plan_describe_workload_lists(zs):
    """Chunk tables for the two model-shaped lists: every element is covered
    exactly once; chunk counts follow from the chunk size."""
    for name in ("gpt2_xl", "llama_7b"):
        wl = W.WORKLOADS[name]
        ents, base = [], 1 << 40
        for _, n in wl.tensors:
            step = (n * 4 + 1023) // 1024 * 1024   # every array on 1 KiB: no head
            ents.append(_fake(n, base, base + step, base + 2 * step, base + 3 * step,
                              base + 4 * step))
            base += 5 * step
        d = zs.zero_plan_describe(ents)
        assert d["n_params"] == wl.n_params and d["n_tensors"] == len(wl.tensors)
        assert d["vector_elems"] + d["scalar_elems"] == wl.n_params
        assert d["scalar_elems"] == sum(n % 4 for _, n in wl.tensors)
        C = d["chunk_elems"]
        assert d["n_chunks"] == sum((n + C - 1) // C for _, n in wl.tensors)
        assert d["table_bytes"] == 64 * len(wl.tensors) + 16 * d["n_chunks"]


def test_plan_heads_of_a_packed_list(zs):
    """The GPT-2-XL list packed into five flattened buffers (each on 1 KiB):
    a tensor at element offset o has fp32 arrays at 4·o bytes past a 1 KiB
    boundary, so a tensor of 1,024 elements or more has a head of
    (256 - o mod 256) mod 256 elements, all by fours (o is a multiple of
    64), and its first chunk holds that head plus up to one chunk.  Chunk
    counts and the vector/single split follow."""
    wl = W.WORKLOADS["gpt2_xl"]
    N = wl.n_params
    bases = [1 << 40, (1 << 40) + 2 * N + 4096, 1 << 42, 1 << 43, 1 << 44]
    bases[1] = (bases[1] + 1023) // 1024 * 1024
    ents, o, heads = [], 0, []
    for _, n in wl.tensors:
        ents.append((bases[0] + 2 * o, bases[1] + 2 * o, bases[2] + 4 * o, bases[3] + 4 * o,
                     bases[4] + 4 * o, n))
        heads.append((256 - o % 256) % 256 if n >= 1024 else 0)
        o += n
    assert sum(1 for h in heads if h) > len(heads) // 2   # most tensors off 1 KiB
    for C in (16384, 4096, 512):
        d = zs.zero_plan_describe(ents, C)
        want = sum(1 + -(-(n - min(n, h + C)) // C) for (_, n), h in zip(wl.tensors, heads))
        assert d["n_chunks"] == want, C
        assert d["scalar_elems"] == sum(n % 4 for _, n in wl.tensors)
        assert d["vector_elems"] + d["scalar_elems"] == N


def _packed(zs, sizes):
    """A would-be plan over tensors packed back to back in five flattened
    buffers that start on 1 KiB."""
    B = [1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44]
    ents, o = [], 0
    for n in sizes:
        ents.append((B[0] + 2 * o, B[1] + 2 * o, B[2] + 4 * o, B[3] + 4 * o, B[4] + 4 * o, n))
        o += n
    return zs.zero_plan_describe(ents)


def test_plan_occupancy_cap(zs):
    """wg_per_cu: 12 with 256-element tiles; with 512-element tiles 7 while
    fewer than one tile in 200 holds a head or a partial last tile, else
    7 * 512 / e + 7 within 14..27 (e: elements per tile with work), 19 and
    21 taken as 20 and 22."""
    d = _packed(zs, [1 << 26])
    assert (d["tile_elems"], d["wg_per_cu"]) == (256, 12)
    d = _packed(zs, [n for _, n in W.WORKLOADS["gpt2_xl"].tensors])
    assert (d["tile_elems"], d["wg_per_cu"]) == (256, 12)
    # whole tiles only: 7
    d = _packed(zs, [1024] * 1000)
    assert (d["tile_elems"], d["wg_per_cu"]) == (512, 7)
    # one partial tile per tensor of 100 elements: e = 100, 7*512/100 + 7 > 27
    d = _packed(zs, [100] * 1000)
    assert (d["tile_elems"], d["wg_per_cu"]) == (512, 27)
    # e = 300: round(7*512/300 + 7) = 19, taken as 20
    assert _packed(zs, [300] * 1000)["wg_per_cu"] == 20
    # e = 250: round(21.3) = 21, taken as 22; e = 200: 24.9 -> 25
    assert _packed(zs, [250] * 1000)["wg_per_cu"] == 22
    assert _packed(zs, [200] * 1000)["wg_per_cu"] == 25
    # e = 400 (tensors of 800: two tiles, one partial): round(8.96 + 7) = 16
    assert _packed(zs, [800] * 1000)["wg_per_cu"] == 16
    # mostly whole tiles: 199 tensors of 512 and one of 100 per 200 tensors
    # (1 irregular tile in 200: the cap moves; 1 in 201 does not)
    assert _packed(zs, ([512] * 199 + [100]) * 5)["wg_per_cu"] == 14
    assert _packed(zs, ([512] * 200 + [100]) * 5)["wg_per_cu"] == 7
    # single-element tensors of whole tiles (m one element off)
    one_off = [((1 << 40) + (k << 20), (1 << 41) + (k << 20), (1 << 42) + (k << 20),
                (1 << 43) + (k << 20) + 4, (1 << 44) + (k << 20), 1024) for k in range(100)]
    d = zs.zero_plan_describe(one_off)
    assert d["scalar_elems"] == 102400 and d["wg_per_cu"] == 7


def test_plan_describe_empty_and_zero_sized(zs):
    d = zs.zero_plan_describe([])
    assert d["n_params"] == 0 and d["n_chunks"] == 0
    d = zs.zero_plan_describe([(0, 0, 0, 0, 0, 0), _fake(10)])
    assert d["n_params"] == 10 and d["n_tensors"] == 2 and d["n_chunks"] == 1


def test_plan_describe_rejects(zs):
    bad = [
        [_fake(10, p=0)],                       # null array of a non-empty tensor
        [_fake(10, p=0x100001)],                # fp16 not 2-byte aligned
        [_fake(10, w=0x300002)],                # fp32 not 4-byte aligned
        [_fake(1000, m=0x300000 + 16)],         # m overlaps master
        [_fake(1000, p=0x200000)],              # param overlaps grad
        [_fake(10), _fake(10, 0x100010, 0x210000, 0x310000, 0x410000, 0x510000)],  # across tensors
    ]
    for ents in bad:
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_plan_describe(ents)
        assert e.value.status == -1
    # gradients are read only: two tensors may share one
    zs.zero_plan_describe([_fake(10), _fake(10, 0x110000, 0x200000, 0x310000, 0x410000, 0x510000)])
    with pytest.raises(zs.ZeroError) as e:
        zs.zero_plan_describe([_fake(2 ** 62, w=2 ** 62)])
    assert e.value.status == -2


def test_step_and_reduce_reject_before_any_device_call(zs):
    _without_devices("_step_and_reduce_reject_before_any_device_call")


def _step_and_reduce_reject_before_any_device_call(zs):
    import ctypes
    L = zs.lib()
    hp = zs.AdamHParams()._c()
    assert L.zero_adam_step(None, ctypes.byref(hp), 1, None, None, None) == -1
    p = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.zero_reduce_grad_shard(p, 0, 8, 0x3000, None, None) == -1
    assert L.zero_reduce_grad_shard(p, 257, 8, 0x3000, None, None) == -1
    assert L.zero_reduce_grad_shard(None, 2, 8, 0x3000, None, None) == -1
    assert L.zero_reduce_grad_shard(p, 2, 8, None, None, None) == -1
    assert L.zero_reduce_grad_shard(p, 2, 8, 0x3001, None, None) == -1     # misaligned out
    assert L.zero_reduce_grad_shard(p, 2, 8, 0x1008, None, None) == -1     # out overlaps a slice
    q = (ctypes.c_void_p * 2)(0x1000, 0)
    assert L.zero_reduce_grad_shard(q, 2, 8, 0x3000, None, None) == -1     # null slice
    # n = 0 with valid pointers returns before launching
    assert L.zero_reduce_grad_shard(p, 2, 0, 0x3000, None, None) == 0


def test_loss_scale_rejects_before_any_device_call(zs):
    _without_devices("_loss_scale_rejects_before_any_device_call")


def _loss_scale_rejects_before_any_device_call(zs):
    """zero_adam_step_scaled and zero_loss_scale_update check their
    pointers and ranges on the host first (fake addresses, never used)."""
    import ctypes
    L = zs.lib()
    hp = zs.AdamHParams()._c()
    S = 0x10000                                   # a fake 16-byte scale record
    assert L.zero_adam_step_scaled(None, ctypes.byref(hp), 1, None, None, None, None) == -1
    assert L.zero_adam_step_scaled(None, ctypes.byref(hp), 1, S, None, None, None) == -1

    def upd(scale=S, flag=0x20000, interval=2000, lo=0, hi=24):
        return L.zero_loss_scale_update(scale, flag, interval, lo, hi, None)

    assert upd(scale=None) == -1
    assert upd(flag=None) == -1
    assert upd(scale=S + 2) == -1                 # misaligned
    assert upd(flag=0x20002) == -1
    for f in (S, S + 4, S + 8, S + 12):           # the flag inside the record
        assert upd(flag=f) == -1
    assert upd(interval=0) == -1
    assert upd(lo=5, hi=4) == -1
    assert upd(lo=-101) == -1
    assert upd(hi=101) == -1
    with pytest.raises(ValueError):
        zs.LossScale(min_log2=3, max_log2=2)
    with pytest.raises(ValueError):
        zs.LossScale(max_log2=101)
    with pytest.raises(ValueError):
        zs.LossScale(interval=0)


def test_fused_rejects_before_any_device_call(zs):
    _without_devices("_fused_rejects_before_any_device_call")


def _fused_rejects_before_any_device_call(zs):
    """zero_reduce_adam_step validates everything on the host first."""
    import ctypes
    L = zs.lib()
    hp = zs.AdamHParams()._c()
    bad_hp = zs.AdamHParams(weight_decay=0.1)._c()
    P = ctypes.c_void_p
    s2 = (P * 2)(0x100000, 0x200000)
    args = dict(param=0x300000, w=0x400000, m=0x500000, v=0x600000)

    def call(sl=s2, nd=2, n=64, param=args["param"], w=args["w"], m=args["m"], v=args["v"],
             gout=None, h=hp, t=1):
        return L.zero_reduce_adam_step(sl, nd, n, param, w, m, v, gout,
                                       ctypes.byref(h) if h is not None else None, t, None, None)

    assert call(sl=None) == -1
    assert call(nd=0) == -1
    assert call(nd=257) == -1
    assert call(h=None) == -1
    assert call(h=bad_hp) == -1
    assert call(t=0) == -1
    assert call(param=None) == -1
    assert call(w=0x400002) == -1                    # fp32 not 4-byte aligned
    assert call(param=0x300001) == -1                # fp16 not 2-byte aligned
    assert call(param=0x100000) == -1                # param is a slice
    assert call(m=0x400000 + 16) == -1               # m overlaps master
    assert call(gout=0x300000 + 8) == -1             # grad_out overlaps param
    assert call(sl=(P * 2)(0x100000, 0)) == -1       # null slice
    assert call(n=2 ** 62) == -2                     # byte counts overflow
    assert call(n=0) == 0                            # nothing to do, no launch
    # two ranks' slices may be the same read-only memory: passes validation
    # (n = 0 stops before any device call)
    assert call(sl=(P * 2)(0x100000, 0x100000), n=0) == 0


def test_comm_volume_matches_oracle(zs, orc):
    for stage in range(4):
        for psi in (0, 1, 7, 1000, 7_500_000_000, 2 ** 40 + 3):
            for nd in (1, 2, 8, 64, 256, 65535):
                for align in (1, 3, 512):
                    got = zs.zero_comm_volume(stage, psi, nd, align)
                    want = orc.comm_volume(stage, psi, nd, align)
                    assert (got["passes"], got["volume_elems"], got["ring_send_elems"]) == \
                        (want["passes"], want["volume"], want["ring_send"]), (stage, psi, nd, align)


def test_comm_volume_rejects(zs, orc):
    import ctypes
    for args in ((4, 10, 2, 1), (0, 10, 0, 1), (0, 10, 2, 0)):
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_comm_volume(*args)
        assert e.value.status == -1
        with pytest.raises(orc.OracleError):
            orc.comm_volume(*args)
    assert zs.lib().zero_comm_volume(0, 10, 2, 1, None) == -1
    # 3 * psi overflows 64 bits in stage 3 only
    psi = 2 ** 63
    zs.zero_comm_volume(1, psi - 1, 1, 1)
    for stage in (0, 3):
        with pytest.raises(zs.ZeroError) as e:
            zs.zero_comm_volume(stage, psi, 1, 1)
        assert e.value.status == -2


def test_gather_rejects_before_any_device_call(zs):
    _without_devices("_gather_rejects_before_any_device_call")


def _gather_rejects_before_any_device_call(zs):
    import ctypes
    L = zs.lib()
    P = ctypes.c_void_p
    S = 64
    full = 0x1000000
    sh = (P * 2)(0x100000, 0x200000)
    assert L.zero_gather_shards(None, 2, S, full, None) == -1
    assert L.zero_gather_shards(sh, 0, S, full, None) == -1
    assert L.zero_gather_shards(sh, 257, S, full, None) == -1
    assert L.zero_gather_shards(sh, 2, S, None, None) == -1
    assert L.zero_gather_shards(sh, 2, S, full + 1, None) == -1                  # misaligned full
    assert L.zero_gather_shards((P * 2)(0x100001, 0x200000), 2, S, full, None) == -1
    assert L.zero_gather_shards((P * 2)(0x100000, 0), 2, S, full, None) == -1   # null shard
    # shard 0 sits inside full but not at its own place (it is shard 1's place)
    assert L.zero_gather_shards((P * 2)(full + 2 * S, 0x200000), 2, S, full, None) == -1
    assert L.zero_gather_shards(sh, 2, 2 ** 63, full, None) == -2
    # nothing to move: zero length, or every shard already in place
    assert L.zero_gather_shards(sh, 2, 0, full, None) == 0
    assert L.zero_gather_shards((P * 2)(full, full + 2 * S), 2, S, full, None) == 0


def test_binding_fails_loudly_without_the_library(tmp_path):
    """A copy of the package without libzeroshard.so: importing the binding
    raises ImportError naming the missing library (no fallback path)."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "zero_partitioned_mixed_layout_amd")
    dst = tmp_path / "zero_partitioned_mixed_layout_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    assert not list(dst.glob("*.so"))
    r = subprocess.run([sys.executable, "-c", "import zero_partitioned_mixed_layout_amd.zero_shard"],
                       cwd=tmp_path, env=dict(os.environ, PYTHONPATH=str(tmp_path)),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libzeroshard.so is missing" in r.stderr


def test_header_is_plain_c_and_links(tmp_path):
    """include/zero_shard.h compiles as strict C99 and C11 with every warning
    an error, and a C program links against the library and calls a host
    entry point through it."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    src = tmp_path / "use.c"
    src.write_text('#include "zero_shard.h"\n'
                   "int main(void) {\n"
                   "    zero_layout l;\n"
                   "    uint64_t b = 0;\n"
                   "    if (zero_shard_layout(7500000000ull, 64, 0, 1, &l) != ZERO_OK) return 1;\n"
                   "    if (l.shard_len != 117187500ull) return 2;\n"
                   "    if (zero_state_bytes(2, 7500000000ull, 64, 1, &b) != ZERO_OK) return 3;\n"
                   "    return b == 16640625000ull ? 0 : 4;\n"
                   "}\n")
    inc = os.path.join(ROOT, "include")
    libdir = os.path.join(ROOT, "zero_partitioned_mixed_layout_amd")
    for std in ("c99", "c11"):
        subprocess.run(["gcc", f"-std={std}", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", inc, "-fsyntax-only", str(src)], check=True, capture_output=True)
    exe = str(tmp_path / "use")
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-L", libdir, "-lzeroshard",
                    f"-Wl,-rpath,{libdir}", "-o", exe], check=True, capture_output=True)
    assert subprocess.run([exe], timeout=120).returncode == 0


def test_noalloc_rejects_before_any_device_call(zs):
    _without_devices("_noalloc_rejects_before_any_device_call")


def _noalloc_rejects_before_any_device_call(zs):
    """zero_adam_step_noalloc checks its arguments and its fixed limits
    (tensor count, table bytes) on the host before it enqueues anything
    (fake addresses, never used)."""
    import ctypes
    L = zs.lib()
    hp = zs.AdamHParams()._c()
    bad_hp = zs.AdamHParams(weight_decay=0.1)._c()
    T = zs._Tensor

    def arr(ts):
        a = (T * max(1, len(ts)))()
        for k, x in enumerate(ts):
            a[k] = x
        return a

    def tensor(base, n):
        # five disjoint arrays spaced 16 n bytes apart
        return T(base, base + 4 * n, base + 8 * n, base + 16 * n, base + 24 * n, n)

    one = [tensor(1 << 30, 1000)]

    def call(ts=one, h=hp, t=1, flag=None, skip=None, n=None):
        a = arr(ts)
        return L.zero_adam_step_noalloc(a, len(ts) if n is None else n,
                                        ctypes.byref(h) if h is not None else None, t, flag,
                                        skip, None)

    assert call(h=None) == -1
    assert call(h=bad_hp) == -1
    assert call(t=0) == -1
    assert call(flag=0x1000, skip=0x1000) == -1          # flag is the skip input
    assert L.zero_adam_step_noalloc(None, 1, ctypes.byref(hp), 1, None, None, None) == -1
    overlap = [tensor(1 << 30, 1000), tensor((1 << 30) + 64, 1000)]
    assert call(ts=overlap) == -1                        # arrays of two tensors overlap
    odd = [T((1 << 30) + 1, 1 << 31, 1 << 32, 1 << 33, 1 << 34, 8)]
    assert call(ts=odd) == -1                            # fp16 array not 2-byte aligned
    assert call(ts=[T(1 << 30, 0, 1 << 32, 1 << 33, 1 << 34, 8)]) == -1   # NULL gradient
    assert call(ts=[tensor(1 << 30, 2 ** 62)]) == -2     # byte counts overflow
    # the fixed limits: more tensors than the array holds descriptors for ...
    many = [tensor((k + 1) << 24, 8) for k in range(zs.ZERO_NOALLOC_MAX_TENSORS + 1)]
    assert call(ts=many) == -6
    # ... and a table past ZERO_NOALLOC_SCRATCH_BYTES: 16384-element chunks
    # of 16 bytes each, one tensor of (2^19 + 1) * 16384 elements
    n_big = ((zs.ZERO_NOALLOC_SCRATCH_BYTES // 16) + 1) * 16384
    big = tensor(1 << 40, n_big)
    assert zs.zero_plan_describe([(big.param_f16, big.grad_f16, big.master, big.m, big.v,
                                   big.n)])["table_bytes"] > \
        zs.ZERO_NOALLOC_SCRATCH_BYTES
    assert call(ts=[tensor(1 << 40, n_big)]) == -6
    # nothing to do: no tensors, or only empty ones, returns before any device call
    assert call(ts=[], n=0) == 0
    assert call(ts=[T(0, 0, 0, 0, 0, 0), T(0, 0, 0, 0, 0, 0)]) == 0
