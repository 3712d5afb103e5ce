"""Pins for the oracle's shard layout and model-state ledger.

Ledger: "The Mathematics" (eq. M_states and M_states(p, N_d)) on the ZeRO and
the Memory Tricks page, the stage table in "The replication nobody
questioned" on the 16-byte-parameter page, and "ZeRO removes replicated state
in stages" on the DeepSpeed ZeRO page.  The printed figures come from
tests/golden/ledger_pages.json, each with its citation.

Layout: ranks own contiguous slices of the flat buffer ("The part that sounds
too good: communication", 16-byte-parameter page).  The padding rule is this
library's reading (tail padding to a multiple of N_d * align elements); it is
pinned by brute force against the properties a partition must have.
"""
import json
import math
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ledger_pages.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _round_sig(x: float, digits: int) -> float:
    if x == 0:
        return 0.0
    return round(x, digits - 1 - int(math.floor(math.log10(abs(x)))))


UNIT = {"GB": 1e9, "GiB": float(2 ** 30)}


@pytest.mark.parametrize("row", _golden()["stage_bytes"],
                         ids=lambda r: f"psi{r['psi']}-nd{r['nd']}-s{r['stage']}-{r['unit']}")
def test_ledger_matches_printed_figures(orc, row):
    b = orc.state_bytes(row["stage"], row["psi"], row["nd"], 1)
    assert _round_sig(b / UNIT[row["unit"]], row["digits"]) == row["printed"], row["cite"]


def test_ledger_exact_bytes_at_7p5b_nd64(orc):
    """Psi = 7.5e9 divides by 64, so the formulas give exact integers."""
    psi = 7_500_000_000
    got = [orc.state_bytes(s, psi, 64) for s in range(4)]
    assert got == [120_000_000_000, 31_406_250_000, 16_640_625_000, 1_875_000_000]


@pytest.mark.parametrize("row", _golden()["fp16_weight_share"], ids=lambda r: str(r["psi"]))
def test_fp16_weights_are_an_eighth_of_state(orc, row):
    """fp16 weights are 12.5% of the 16-byte ledger."""
    share = _golden()["shares"]["fp16_weights_percent"] / 100
    b = orc.state_bytes(0, row["psi"], 1) * share
    assert _round_sig(b / UNIT[row["unit"]], row["digits"]) == row["printed"], row["cite"]


def test_optimizer_share_and_stage_limits(orc):
    """As N_d grows, stage 1 keeps only the 4 replicated bytes (fp16 param +
    grad) and stage 2 only the 2 bytes of fp16 params: cuts of 4x and 8x;
    the optimizer's K = 12 bytes are 75% of the ledger; stage 3 is 16/N_d."""
    g = _golden()
    psi = 1 << 40
    full = orc.state_bytes(0, psi, 1)
    nd = 1 << 20
    s1 = orc.state_bytes(1, psi, nd)
    s2 = orc.state_bytes(2, psi, nd)
    assert abs(full / s1 - g["limits"]["stage1_cut"]) < 1e-4
    assert abs(full / s2 - g["limits"]["stage2_cut"]) < 1e-4
    # what stage 1 stops replicating is the optimizer's share
    assert (full - s1) / full == pytest.approx(g["shares"]["optimizer_percent"] / 100, abs=1e-4)
    # stage 3 is linear in N_d: doubling the ranks halves the bytes
    for k in range(0, 20):
        assert orc.state_bytes(3, psi, 1 << k) == 2 * orc.state_bytes(3, psi, 1 << (k + 1))
    # the cuts grow monotonically toward their limits
    prev1 = prev2 = 0
    for k in range(0, 12):
        c1 = full / orc.state_bytes(1, psi, 1 << k)
        c2 = full / orc.state_bytes(2, psi, 1 << k)
        assert prev1 < c1 < 4 and prev2 < c2 < 8 or k == 0
        prev1, prev2 = c1, c2


def test_ledger_identities(orc):
    """One rank (N_d = 1) holds the whole 16 Psi at every stage; N_d times the
    stage-3 bytes is 16 Psi when N_d divides Psi."""
    for psi in (0, 1, 7, 1000, 1_557_611_200, 6_738_415_616, 7_500_000_000):
        for s in range(4):
            assert orc.state_bytes(s, psi, 1) == 16 * psi
        for nd in (1, 2, 4, 8, 64):
            if psi % nd == 0:
                assert nd * orc.state_bytes(3, psi, nd) == 16 * psi


def test_ledger_counts_padding(orc):
    """A rank allocates a padded shard: S = padded_total / N_d."""
    psi, nd, align = 7_500_000_000, 8, 512
    S = 937_500_160
    assert orc.state_bytes(1, psi, nd, align) == 4 * psi + 12 * S
    assert orc.state_bytes(2, psi, nd, align) == 2 * psi + 14 * S
    assert orc.state_bytes(3, psi, nd, align) == 16 * S
    assert orc.state_bytes(0, psi, nd, align) == 16 * psi


def test_ledger_rejects(orc):
    with pytest.raises(orc.OracleError):
        orc.state_bytes(4, 10, 1)
    with pytest.raises(orc.OracleError):
        orc.state_bytes(0, 10, 0)
    with pytest.raises(orc.OracleError):           # 16 Psi overflows 64 bits
        orc.state_bytes(0, 1 << 61, 1)


def test_layout_workload_shards(orc):
    """The shard sizes the workloads state: 262,144 of 2^20 over 4 ranks;
    117.19M of 7.5e9 over 64; 937.5M of 7.5e9 over 8 in 512-element units."""
    assert orc.shard_layout(2 ** 20, 4, 0, 1) == dict(
        padded_total=2 ** 20, shard_len=262_144, offset=0, real_len=262_144)
    assert orc.shard_layout(7_500_000_000, 64, 0, 1)["shard_len"] == 117_187_500
    assert orc.shard_layout(7_500_000_000, 64, 63, 1)["offset"] == 63 * 117_187_500
    l3 = orc.shard_layout(7_500_000_000, 8, 3, 512)
    assert l3 == dict(padded_total=7_500_001_280, shard_len=937_500_160,
                      offset=2_812_500_480, real_len=937_500_160)
    l7 = orc.shard_layout(7_500_000_000, 8, 7, 512)
    assert l7["real_len"] == 937_498_880 and l7["offset"] == 6_562_501_120


def test_layout_brute_force_partition(orc):
    """For every small (Psi, N_d, align): the real parts of the shards tile
    [0, Psi) in rank order without gaps or overlap, every shard has the same
    length, a multiple of align, and padding is less than one N_d*align unit."""
    for psi in range(0, 301):
        for nd in range(1, 10):
            for align in (1, 2, 3, 8, 512):
                lays = [orc.shard_layout(psi, nd, r, align) for r in range(nd)]
                P = lays[0]["padded_total"]
                S = lays[0]["shard_len"]
                assert all(l["padded_total"] == P and l["shard_len"] == S for l in lays)
                assert P % (nd * align) == 0 and P >= psi and P - psi < nd * align
                assert S * nd == P and S % align == 0
                pos = 0
                for r, l in enumerate(lays):
                    assert l["offset"] == r * S
                    if l["real_len"]:
                        assert l["offset"] == pos
                    pos += l["real_len"]
                    assert 0 <= l["real_len"] <= S
                    assert l["real_len"] == max(0, min(S, psi - l["offset"]))
                assert pos == psi
                # every element index belongs to exactly one rank
                owner = [i // S for i in range(psi)] if S else []
                assert all(0 <= o < nd for o in owner)


def test_layout_rejects(orc):
    for args in ((10, 0, 0, 1), (10, 4, 4, 1), (10, 4, 0, 0)):
        with pytest.raises(orc.OracleError):
            orc.shard_layout(*args)
    with pytest.raises(orc.OracleError):            # padded total overflows
        orc.shard_layout(2 ** 64 - 1, 3, 0, 512)
    assert orc.shard_layout(2 ** 64 - 1, 1, 0, 1)["shard_len"] == 2 ** 64 - 1
