"""Pins for the oracle's layout, schedule and combine plan (CPU only).

What pins what (none re-derives the plan with the plan's own formulas):
* Figures 2b and 2c of the tile-signal notes as hand-worked fixtures
  (tests/golden) -> layout order, padding position, rule (ii), rule (i),
  receive offsets, segments, owner-side slots.
* The padding figures printed in §4.3 and §11.10 -> padding bound.
* A sort-based layout (oracle.brute.layout_by_sorting, no histogram or
  scan) on random small routings -> grouping, group order, padding.
* Tightness of the bound on groups of size 1 mod tb_M.
* All ranks' plans together must write every row of every owner's receive
  buffer exactly once, and a label payload must arrive where the owner's
  slot table looks for it -> receive bases, dst_off, valid, pos.
* Special cases: tb_M = 1 (no padding), W = 1 (no remote bands: plain
  grouped FFN), local group empty, all rows from one owner, r = W - 1.
* The invariants module on every named workload's plan.
"""
import json
import os

import numpy as np
import pytest

from oracle import plan as P
from oracle import brute, invariants
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def _check_bands(pl, expected):
    b = pl.bands
    assert pl.n_bands == len(expected)
    for s, exp in enumerate(expected):
        for key, val in exp.items():
            assert int(b[key][s]) == val, (s, key, int(b[key][s]), val)


def test_fig2b_layout():
    g = load("fig2b_layout.json")
    pl = P.build_plan(np.array(g["topk_ids"]), g["tokens"], g["rank"], g["E_l"], g["tb_m"])
    ex = g["expected"]
    assert pl.c.tolist() == ex["c"]
    assert pl.m_e.tolist() == ex["m_e"]
    assert pl.src_index.tolist() == ex["src_index"]
    assert pl.n_remote == ex["n_remote"]
    _check_bands(pl, ex["bands_in_schedule_order"])
    invariants.check(pl)


def test_fig2c_schedule():
    g = load("fig2c_schedule.json")
    pl = P.build_plan(np.array(g["topk_ids"]), g["tokens"], g["rank"], g["E_l"], g["tb_m"])
    ex = g["expected"]
    assert pl.src_index.tolist() == ex["src_index"]
    assert pl.row_off.tolist() == ex["row_off"]
    assert pl.rb.tolist() == ex["rb"]
    assert pl.expert_order.tolist() == ex["expert_order"]
    assert pl.n_remote == ex["n_remote"]
    _check_bands(pl, ex["bands_in_schedule_order"])
    assert pl.segs["first_band"].tolist() == ex["segments_mgb1_first_band"]
    assert pl.n_remote_segs == ex["n_remote_segments"]
    assert pl.pos.tolist() == ex["pos"]
    invariants.check(pl)


def test_padding_figures_from_the_notes():
    g = load("padding_pins.json")
    for case in g["cases"]:
        assert P.padding_bound(case["W"], case["tb_m"]) == case["bound"]
        if "percent" in case:
            assert round(100.0 * case["bound"] / case["rows"], 2) == case["percent"]


@pytest.mark.parametrize("W,tb", [(2, 4), (4, 8), (5, 3), (8, 16)])
def test_padding_bound_is_reached(W, tb):
    # every remote owner sends 1 (mod tb) rows to local expert 0 of rank 0
    E_l, k, r = 1, 1, 0
    tokens = [tb + 1] * W
    ids = np.zeros((sum(tokens), k), dtype=np.int32)   # all to global expert 0
    pl = P.build_plan(ids, tokens, r, E_l, tb)
    assert int(pl.m_e[0]) - pl.R == P.padding_bound(W, tb)
    invariants.check(pl)


def _random_cases(n, seed=1):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        W = int(rng.integers(1, 6))
        E_l = int(rng.integers(1, 5))
        E = W * E_l
        k = int(rng.integers(1, min(E, 4) + 1))
        tokens = [int(rng.integers(0, 12)) for _ in range(W)]
        tb = int(rng.choice([1, 2, 3, 4, 8]))
        r = int(rng.integers(0, W))
        mgb = int(rng.integers(1, 4))
        hot = int(rng.integers(0, E)) if rng.random() < 0.5 else None
        ids = synth.random_routing_case(rng, W, E_l, k, tokens, hot=hot)
        yield ids, tokens, r, E_l, tb, mgb


def test_layout_matches_sorting_definition():
    for ids, tokens, r, E_l, tb, mgb in _random_cases(150):
        pl = P.build_plan(ids, tokens, r, E_l, tb, mgb)
        ref = brute.layout_by_sorting(ids, tokens, r, E_l, tb)
        for e in range(E_l):
            got = pl.src_index[pl.row_off[e]:pl.row_off[e + 1]].tolist()
            assert got == ref[e], (tokens, r, E_l, tb, e)
        invariants.check(pl)


def test_all_ranks_tile_every_receive_buffer_once():
    """Over the W ranks' plans, each owner row is written exactly once, and a
    label payload (owner, token, expert) reaches the slot the owner's pos
    table reads for that (token, slot)."""
    for ids, tokens, _, E_l, tb, mgb in _random_cases(80, seed=2):
        W = len(tokens)
        k = ids.shape[1]
        off = P.owner_offsets(tokens)
        writes = [np.zeros(tokens[o] * k, dtype=np.int64) for o in range(W)]
        label = [np.full((tokens[o] * k, 3), -1, dtype=np.int64) for o in range(W)]
        for r in range(W):
            pl = P.build_plan(ids, tokens, r, E_l, tb, mgb)
            b = pl.bands
            for s in range(pl.n_bands):
                for q in range(int(b["valid"][s])):
                    row = int(b["src_row"][s]) + q
                    i = int(pl.src_index[row])
                    o = int(pl.recv_owner[i])
                    dst = int(b["dst_off"][s]) + q
                    assert o == int(b["dst"][s])
                    writes[o][dst] += 1
                    label[o][dst] = (o, int(pl.recv_token[i]), r * E_l + int(pl.recv_expert[i]))
        for o in range(W):
            assert np.all(writes[o] == 1)
            pl_o = P.build_plan(ids, tokens, o, E_l, tb, mgb)
            for t in range(tokens[o]):
                for j in range(k):
                    got = tuple(label[o][pl_o.pos[t, j]])
                    assert got == (o, t, int(ids[off[o] + t, j]))


def test_tb1_has_no_padding():
    for ids, tokens, r, E_l, _, mgb in _random_cases(30, seed=3):
        pl = P.build_plan(ids, tokens, r, E_l, 1, mgb)
        assert pl.M == pl.R
        assert np.all(pl.src_index >= 0)


def test_single_rank_is_a_plain_grouped_layout():
    # W = 1: no remote rows, the layout is the rows grouped by expert in
    # arrival order, and every band is local
    rng = np.random.default_rng(4)
    ids = synth.random_routing_case(rng, 1, 4, 2, [40])
    pl = P.build_plan(ids, [40], 0, 4, 8)
    assert pl.n_remote == 0 and pl.n_remote_segs == 0
    flat = ids.reshape(-1)
    expect = np.concatenate([np.nonzero(flat == e)[0] for e in range(4)])
    assert pl.src_index.tolist() == expect.tolist()


def test_empty_local_group_and_single_owner():
    W, E_l, k, tb = 3, 2, 1, 4
    tokens = [5, 3, 2]
    # every token goes to global expert 0 (rank 0); rank 0's own tokens too
    ids = np.zeros((sum(tokens), k), dtype=np.int32)
    pl = P.build_plan(ids, tokens, 0, E_l, tb)
    assert pl.c[:, 0].tolist() == [5, 0]
    assert pl.m_e.tolist() == [4 + 4 + 5, 0]
    invariants.check(pl)
    # only owner 2 routes anything to rank 1, and rank 1's local group is empty
    ids2 = np.full((sum(tokens), k), 0, dtype=np.int32)
    ids2[8:10] = 3
    pl2 = P.build_plan(ids2, tokens, 1, E_l, tb)
    assert pl2.c.tolist() == [[0, 0, 0], [0, 0, 2]]
    assert pl2.m_e.tolist() == [0, 4]
    assert pl2.n_remote == 1 and pl2.n_bands == 1
    invariants.check(pl2)


def test_last_rank_and_k_equals_E():
    W, E_l = 3, 1
    tokens = [3, 2, 4]
    ids = np.tile(np.arange(3, dtype=np.int32), (sum(tokens), 1))
    pl = P.build_plan(ids, tokens, W - 1, E_l, 2)
    assert pl.c.tolist() == [[3, 2, 4]]
    assert pl.grp_off.tolist() == [[0, 4, 6]]
    invariants.check(pl)


@pytest.mark.parametrize("name", ["tiny", "mixtral", "qwen3", "dsv3_skew", "decode_tb32", "decode_tb64"])
def test_named_workload_plans_satisfy_invariants(name):
    cfg = synth.get_config(name)
    ids, _ = synth.routing(cfg)
    for mgb in (1, 2):
        pl = P.build_plan(ids, cfg.tokens, cfg.rank, cfg.E_l, cfg.tb_m, mgb)
        invariants.check(pl)


def test_segments_mgb_runs():
    # one remote group of 7 bands: [0], [1,2], [3,4], [5], [6] with mgb = 2
    W, E_l, tb = 2, 1, 1
    tokens = [7, 0]
    ids = np.ones((7, 1), dtype=np.int32)        # owner 0 -> global expert 1 (rank 1)
    pl = P.build_plan(ids, tokens, 1, E_l, tb, mgb=2)
    assert pl.segs["first_band"].tolist() == [0, 1, 3, 5, 6]
    assert pl.segs["n_bands"].tolist() == [1, 2, 2, 1, 1]
    assert pl.segs["rows"].tolist() == [1, 2, 2, 1, 1]
    pl3 = P.build_plan(ids, tokens, 1, E_l, tb, mgb=3)
    assert pl3.segs["n_bands"].tolist() == [1, 3, 2, 1]
