"""Negative pins of ``oracle.invariants`` (CPU only).

A valid plan passes; each test then plants one plausible builder mistake in a
copy of that plan and checks that the property it breaks is reported by name
(tile-signal notes §4.2 layout, §4.3 padding bound, §4.4 rules (i) and (ii),
§4.5 combine plan, §5.2 segments).  So no check is vacuous: a silent pass of
``invariants.check`` on the GPU's or the oracle's plans means something.
"""
import copy

import numpy as np
import pytest

import synth
from oracle import invariants
from oracle import plan as P

W, E_L, K, TB, MGB, RANK = 4, 3, 2, 8, 2, 1
TOKENS = [61, 93, 47, 72]


@pytest.fixture(scope="module")
def base():
    rng = np.random.default_rng(7)
    ids = synth.random_routing_case(rng, W, E_L, K, TOKENS)
    pl = P.build_plan(ids, TOKENS, RANK, E_L, TB, MGB)
    # the mutations below need these features of the plan
    assert invariants.violations(pl) == []
    assert pl.n_remote >= 4 and pl.n_bands > pl.n_remote
    assert np.any((pl.c[:, [o for o in range(W) if o != RANK]] % TB) != 0)
    assert np.all(pl.c[:, RANK] > 0)
    assert len(set(pl.rb.tolist())) > 1
    assert np.any(pl.segs["n_bands"] > 1)
    return pl


def clone(pl):
    return copy.deepcopy(pl)


def insert_rows(pl, e, at, n):
    """Insert n padding rows into X_e before layout row `at` (at most X_e's
    end), shifting every later row (X_e starts, band and segment source
    rows)."""
    q = clone(pl)
    assert q.row_off[e] <= at <= q.row_off[e + 1]
    q.src_index = np.concatenate([q.src_index[:at], np.full(n, -1, np.int64), q.src_index[at:]])
    q.row_off = q.row_off.copy()
    q.row_off[e + 1:] += n
    q.m_e = np.diff(q.row_off)
    for arr in (q.bands["src_row"], q.segs["src_row"]):
        arr[arr >= at] += n
    return q


def group_start(pl, e, o):
    return int(pl.row_off[e] + pl.grp_off[e, o])


def remote_owners():
    return [o for o in range(W) if o != RANK]


def expect(pl, name):
    v = invariants.violations(pl)
    assert name in v, (name, v)
    with pytest.raises(AssertionError, match=name):
        invariants.check(pl)


def test_valid_plans_pass(base):
    invariants.check(base)
    for name in ["tiny", "mixtral", "decode_tb32"]:
        cfg = synth.get_config(name)
        ids, _ = synth.routing(cfg)
        invariants.check(P.build_plan(ids, cfg.tokens, cfg.rank, cfg.E_l, cfg.tb_m, cfg.mgb))


def test_padding_the_local_group(base):
    e = 0
    end = group_start(base, e, RANK) + int(base.c[e, RANK])
    expect(insert_rows(base, e, end, TB - 1), "local-group-padded")


def test_padding_beyond_the_next_multiple(base):
    e = 0
    o = remote_owners()[0]
    end = group_start(base, e, o) + P.padded(int(base.c[e, o]), TB)
    expect(insert_rows(base, e, end, TB), "padding-not-minimal")


def test_padding_bound_per_expert_and_rank(base):
    q = base
    for e in range(E_L):
        for o in remote_owners():
            # a builder that pads every group by one more band than needed
            end = group_start(q, e, o) + P.padded(int(q.c[e, o]), TB)
            q = insert_rows(q, e, end, TB)
    v = invariants.violations(q)
    assert "padding-bound-expert" in v and "padding-bound-rank" in v, v


def test_local_band_before_a_remote_band(base):
    q = clone(base)
    i, j = q.n_remote - 1, q.n_remote
    for f in q.bands:
        q.bands[f][[i, j]] = q.bands[f][[j, i]]
    expect(q, "remote-after-local")


def test_rule_ii_order(base):
    q = clone(base)
    nr = q.n_remote
    ex = q.bands["expert"][:nr]
    last = ex[-1]
    # move the remote bands of the last expert (the fewest remote bands) to the front
    perm = np.concatenate([np.nonzero(ex == last)[0], np.nonzero(ex != last)[0], np.arange(nr, q.n_bands)])
    assert q.rb[last] < q.rb[ex[0]]
    for f in q.bands:
        q.bands[f] = q.bands[f][perm]
    expect(q, "rule-ii")


def test_remote_bands_of_an_expert_split(base):
    q = clone(base)
    nr = q.n_remote
    ex = q.bands["expert"][:nr]
    i = 0
    j = int(np.nonzero(ex != ex[0])[0][0])   # first band of the second expert
    k = int(np.nonzero(ex == ex[0])[0][-1])  # last band of the first expert
    assert k > i
    perm = np.arange(q.n_bands)
    perm[[k, j]] = perm[[j, k]]
    for f in q.bands:
        q.bands[f] = q.bands[f][perm]
    expect(q, "remote-bands-not-contiguous")


def test_padding_row_sent(base):
    q = clone(base)
    s = int(np.nonzero((q.bands["remote"] == 1) & (q.bands["valid"] < TB))[0][0])
    q.bands["valid"][s] += 1
    expect(q, "padding-sent")
    expect(q, "padding-inside-valid")


def test_overlapping_destination_intervals(base):
    q = clone(base)
    b = q.bands
    o = int(b["dst"][0])
    same = np.nonzero(b["dst"] == o)[0]
    assert same.size >= 2
    b["dst_off"][same[1]] = b["dst_off"][same[0]]
    expect(q, "overlapping-writes")


def test_row_dropped_from_the_plan(base):
    q = clone(base)
    s = int(np.nonzero(q.bands["valid"] > 1)[0][0])
    q.bands["valid"][s] -= 1
    expect(q, "group-coverage")
    expect(q, "row-not-sent-once")


def test_band_with_two_owners(base):
    q = clone(base)
    b = q.bands
    s0 = 0
    s1 = int(np.nonzero(b["dst"] != b["dst"][0])[0][0])
    r0, r1 = int(b["src_row"][s0]), int(b["src_row"][s1])
    q.src_index[[r0, r1]] = q.src_index[[r1, r0]]
    expect(q, "mixed-owners")


def test_band_with_a_wrong_expert(base):
    q = clone(base)
    q.bands["expert"][0] = (q.bands["expert"][0] + 1) % E_L
    expect(q, "wrong-expert")


def test_band_valid_out_of_range(base):
    q = clone(base)
    q.bands["valid"][0] = TB + 1
    expect(q, "band-valid-range")


def test_remote_band_tail_holds_a_row(base):
    q = clone(base)
    s = int(np.nonzero((q.bands["remote"] == 1) & (q.bands["valid"] < TB))[0][0])
    q.src_index[int(q.bands["src_row"][s] + q.bands["valid"][s])] = 0
    expect(q, "remote-tail-not-padding")


def test_remote_groups_out_of_rank_order(base):
    q = clone(base)
    ro = remote_owners()
    for e in range(E_L):
        for a in range(len(ro)):
            for b in range(a + 1, len(ro)):
                oa, ob = ro[a], ro[b]
                na, nb = P.padded(int(q.c[e, oa]), TB), P.padded(int(q.c[e, ob]), TB)
                if na == nb and na > 0:
                    sa, sb = group_start(q, e, oa), group_start(q, e, ob)
                    blk = q.src_index[sa:sa + na].copy()
                    q.src_index[sa:sa + na] = q.src_index[sb:sb + nb]
                    q.src_index[sb:sb + nb] = blk
                    expect(q, "group-order")
                    return
    pytest.fail("no two remote groups of equal padded size")


def greedy_segments_without_first_last_rule(pl, mgb):
    """A plausible segment-builder mistake: greedy runs of <= mgb bands of one
    group over the whole band list, with no single-band first and last
    remote segment."""
    b = pl.bands
    runs, cur = [], []
    for s in range(pl.n_bands):
        key = (int(b["expert"][s]), int(b["dst"][s]))
        if cur and (len(cur) == mgb or key != (int(b["expert"][cur[-1]]), int(b["dst"][cur[-1]]))
                    or (s == pl.n_remote)):
            runs.append(cur)
            cur = []
        cur.append(s)
    if cur:
        runs.append(cur)
    n_rs = sum(1 for r in runs if r[0] < pl.n_remote)
    segs = {"first_band": [], "n_bands": [], "dst": [], "dst_off": [], "src_row": [], "rows": []}
    for r in runs:
        segs["first_band"].append(r[0])
        segs["n_bands"].append(len(r))
        segs["dst"].append(int(b["dst"][r[0]]))
        segs["dst_off"].append(int(b["dst_off"][r[0]]))
        segs["src_row"].append(int(b["src_row"][r[0]]))
        segs["rows"].append(int(sum(int(b["valid"][s]) for s in r)))
    return {k: np.array(v, np.int64) for k, v in segs.items()}, n_rs


def test_first_and_last_segment_rule():
    # a routing whose first remote group spans several bands and whose last
    # remote group spans an even number of them (so plain greedy pairs
    # merge the last band with the one before it)
    tokens = [120, 150, 130, 140]
    for seed in range(50):
        rng = np.random.default_rng(seed)
        ids = synth.random_routing_case(rng, W, E_L, K, tokens)
        pl = P.build_plan(ids, tokens, RANK, E_L, TB, MGB)
        b = pl.bands
        key = lambda s: (int(b["expert"][s]), int(b["dst"][s]))
        nr = pl.n_remote
        first = sum(1 for s in range(nr) if key(s) == key(0))
        last = sum(1 for s in range(nr) if key(s) == key(nr - 1))
        if first >= 2 and last >= 2 and last % 2 == 0:
            break
    else:
        pytest.fail("no suitable routing")
    invariants.check(pl)
    q = clone(pl)
    q.segs, q.n_remote_segs = greedy_segments_without_first_last_rule(pl, MGB)
    v = invariants.violations(q)
    assert "first-segment" in v and "last-segment" in v, v


def test_segment_longer_than_mgb(base):
    q = clone(base)
    q.mgb = 1
    expect(q, "segment-too-long")


def test_segment_across_groups(base):
    q = clone(base)
    sg = q.segs
    b = q.bands
    for i in range(sg["first_band"].shape[0] - 1):
        s_last = int(sg["first_band"][i] + sg["n_bands"][i] - 1)
        s_next = int(sg["first_band"][i + 1])
        if (b["expert"][s_last], b["dst"][s_last]) != (b["expert"][s_next], b["dst"][s_next]) and \
                sg["n_bands"][i] + sg["n_bands"][i + 1] <= MGB:
            sg["n_bands"][i] += sg["n_bands"][i + 1]
            sg["rows"][i] += sg["rows"][i + 1]
            for f in sg:
                sg[f] = np.delete(sg[f], i + 1)
            expect(q, "segment-crosses-group")
            return
    pytest.fail("no two adjacent single-band segments of different groups")


def test_segment_offsets_and_rows(base):
    q = clone(base)
    q.segs["dst_off"][1] += 1
    expect(q, "segment-not-contiguous")
    q = clone(base)
    q.segs["rows"][1] += 1
    expect(q, "segment-rows")


def test_segment_missing(base):
    q = clone(base)
    for f in q.segs:
        q.segs[f] = np.delete(q.segs[f], 2)
    expect(q, "segments-do-not-tile")
