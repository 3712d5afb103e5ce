"""Pins for the oracle's communication ledger and parameter gather.

Volumes: "The part that sounds too good: communication" on the
16-byte-parameter page and the stage table in "What It Enabled" on the ZeRO
and the Memory Tricks page (tests/golden/comm_pages.json, each figure with
its citation).  The per-rank ring counts are pinned by simulating ring
reduce-scatters and all-gathers message by message in exact integer
arithmetic.  The gather is pinned by that simulation and by the property the
pages' stage-2 description implies: N_d ranks that each reduce their own
partition of the gradients, update only their slice and all-gather the fp16
parameters end with exactly the state of one plain data-parallel step.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "comm_pages.json")
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("row", _golden()["volume_in_psi"], ids=lambda r: f"stage{r['stage']}")
def test_volume_matches_printed_multiples_of_psi(orc, row):
    for psi, nd in ((7_500_000_000, 64), (1_500_000_000, 8), (1000, 1), (12345, 7)):
        c = orc.comm_volume(row["stage"], psi, nd, 1)
        assert c["volume"] == row["printed"] * psi
        assert c["passes"] == row["printed"]


def test_stage3_ratio(orc):
    want = _golden()["stage3_ratio"]["printed"]
    for psi in (7_500_000_000, 10 ** 6 + 3):
        base = orc.comm_volume(0, psi, 8, 1)["volume"]
        for stage in (1, 2):
            assert orc.comm_volume(stage, psi, 8, 1)["volume"] == base
        assert orc.comm_volume(3, psi, 8, 1)["volume"] == want * base


def _ring_reduce_scatter(data, S):
    """data[r]: rank r's full list of ints (nd * S).  At step k rank r sends
    its running sum of chunk (r - k - 1) mod nd to rank r + 1, which adds it
    into its own copy.  Returns (per-rank element counts sent, data), after
    which rank r holds the complete sum of chunk r."""
    nd = len(data)
    sent = [0] * nd
    for k in range(nd - 1):
        msgs = []
        for r in range(nd):
            c = (r - k - 1) % nd
            msgs.append(((r + 1) % nd, c, data[r][c * S:(c + 1) * S]))
            sent[r] += S
        for dst, c, chunk in msgs:
            for i, x in enumerate(chunk):
                data[dst][c * S + i] += x
    return sent, data


def _ring_all_gather(owned, S):
    """owned[r]: rank r's chunk r.  At step k rank r sends chunk (r - k) mod
    nd to rank r + 1.  Returns (per-rank counts sent, every rank's buffer)."""
    nd = len(owned)
    buf = [[None] * (nd * S) for _ in range(nd)]
    for r in range(nd):
        buf[r][r * S:(r + 1) * S] = owned[r]
    sent = [0] * nd
    for k in range(nd - 1):
        msgs = []
        for r in range(nd):
            c = (r - k) % nd
            msgs.append(((r + 1) % nd, c, buf[r][c * S:(c + 1) * S]))
            sent[r] += S
        for dst, c, chunk in msgs:
            assert None not in chunk
            buf[dst][c * S:(c + 1) * S] = chunk
    return sent, buf


@pytest.mark.parametrize("nd", [1, 2, 3, 4, 5, 8])
def test_ring_counts_and_data(orc, nd):
    """Every rank sends (nd - 1) * S elements per ring pass; the ring
    reduce-scatter leaves rank r the sum of partition r, the all-gather
    leaves every rank the concatenation (the oracle's gather)."""
    rng = np.random.default_rng(nd)
    for psi, align in ((0, 1), (1, 1), (7, 1), (100, 3), (257, 8)):
        lay = orc.shard_layout(psi, nd, 0, align)
        P, S = lay["padded_total"], lay["shard_len"]
        data = [[int(x) for x in rng.integers(0, 1000, P)] for _ in range(nd)]
        total = [sum(d[i] for d in data) for i in range(P)]
        sent_rs, red = _ring_reduce_scatter([list(d) for d in data], S)
        owned = [red[r][r * S:(r + 1) * S] for r in range(nd)]
        for r in range(nd):
            assert owned[r] == total[r * S:(r + 1) * S]
        sent_ag, full = _ring_all_gather(owned, S)
        g = orc.gather([np.array(o, dtype=np.uint16) for o in owned]) if P else np.zeros(0)
        for r in range(nd):
            assert full[r] == [int(x) for x in g]
        per_pass = sent_rs[0]
        assert all(s == per_pass for s in sent_rs + sent_ag)
        for stage in range(4):
            c = orc.comm_volume(stage, psi, nd, align)
            assert c["ring_send"] == c["passes"] * per_pass == c["passes"] * (nd - 1) * S


def test_gather_is_concatenation_and_rejects(orc):
    rng = np.random.default_rng(3)
    for nd, S in ((1, 5), (3, 0), (4, 7), (16, 33)):
        shards = [rng.integers(0, 1 << 16, S).astype(np.uint16) for _ in range(nd)]
        assert np.array_equal(orc.gather(shards), np.concatenate(shards) if S else np.zeros(0))
    with pytest.raises(orc.OracleError):
        orc.comm_volume(4, 10, 2, 1)
    with pytest.raises(orc.OracleError):
        orc.comm_volume(0, 10, 0, 1)


@pytest.mark.parametrize("psi,nd,align", [(1000, 4, 1), (1003, 8, 3), (517, 3, 8), (1, 2, 1),
                                          (64, 64, 1), (300, 7, 5), (4096, 1, 1)])
def test_zero_stage2_step_equals_data_parallel_step(orc, psi, nd, align):
    """Plain data parallelism: all-reduce (mean over ranks) the full fp16
    gradients, every rank updates the whole state.  ZeRO stage 2: rank q
    reduces only its partition, updates only its shard, then the fp16 shards
    are all-gathered.  The resulting fp16 parameters, master, m and v are
    identical bit for bit, padding included."""
    rng = np.random.default_rng(psi + nd)
    lay = orc.shard_layout(psi, nd, 0, align)
    P, S = lay["padded_total"], lay["shard_len"]
    grads = []
    for _ in range(nd):
        g = np.zeros(P, np.float64)
        g[:psi] = rng.standard_normal(psi) * 1e-3
        grads.append(g.astype(np.float16).view(np.uint16))
    w0 = (rng.standard_normal(P) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(P) * 1e-4).astype(np.float32)
    v0 = (rng.random(P) * 1e-6).astype(np.float32)
    t = 4
    # data parallel
    g_dp, f_dp = orc.reduce_grad(grads)
    p_dp = np.zeros(P, np.uint16)
    w_dp, m_dp, v_dp = w0.copy(), m0.copy(), v0.copy()
    a_dp = orc.adam_step(g_dp, p_dp, w_dp, m_dp, v_dp, t=t, **HP)
    # ZeRO stage 2 over nd simulated ranks
    shards_p, shards_w, shards_m, shards_v, flags = [], [], [], [], 0
    for q in range(nd):
        lq = orc.shard_layout(psi, nd, q, align)
        lo, hi = lq["offset"], lq["offset"] + lq["shard_len"]
        assert hi - lo == S
        g_q, f_q = orc.reduce_grad([g[lo:hi] for g in grads])
        p_q = np.zeros(S, np.uint16)
        w_q, m_q, v_q = w0[lo:hi].copy(), m0[lo:hi].copy(), v0[lo:hi].copy()
        flags |= f_q | orc.adam_step(g_q, p_q, w_q, m_q, v_q, t=t, **HP)
        shards_p.append(p_q)
        shards_w.append(w_q)
        shards_m.append(m_q)
        shards_v.append(v_q)
    assert np.array_equal(orc.gather(shards_p), p_dp)
    for parts, ref in ((shards_w, w_dp), (shards_m, m_dp), (shards_v, v_dp)):
        assert np.array_equal(np.concatenate(parts).view(np.uint32), ref.view(np.uint32))
    assert flags == (f_dp | a_dp)
