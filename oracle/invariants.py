"""Properties the pages fix for layout, schedule and combine plan (test
infrastructure only).  Each check raises AssertionError with a message.

* tile-signal notes §4.2: every full-height band has exactly one owner
  (destination rank); padding sits only at the end of remote groups and is the
  minimum that reaches a multiple of tb_M;
* §4.3 / §4.5: padding of one X_e is at most (W-1)(tb_M-1) rows;
* §4.2 step 2 / §4.5: padding rows are never sent;
* §4.4 rule (i): remote bands precede local bands; rule (ii): along the remote
  prefix the experts appear in non-increasing order of remote band count;
* §4.5: the write intervals of one rank's plan are disjoint within every
  owner's receive buffer and cover exactly the group's rows;
* §5.2: the first and the last remote segment are single bands, the others
  hold at most mgb bands; a segment is contiguous at both ends.
"""
from __future__ import annotations

import numpy as np

from .plan import padding_bound


def check(plan, topk_ids=None) -> None:
    W, r, tb = plan.W, plan.r, plan.tb_m
    b = plan.bands
    B = plan.n_bands
    src = plan.src_index

    # one owner per band, padding only at the end of remote bands
    for s in range(B):
        lo = int(b["src_row"][s])
        v = int(b["valid"][s])
        rows = src[lo:lo + v]
        assert np.all(rows >= 0), f"band {s}: padding inside the valid rows"
        owners = plan.recv_owner[rows]
        assert np.all(owners == b["dst"][s]), f"band {s}: mixed owners"
        assert np.all(plan.recv_expert[rows] == b["expert"][s]), f"band {s}: wrong expert"
        if b["remote"][s]:
            assert np.all(src[lo + v:lo + tb] == -1), f"band {s}: remote band tail is not padding"
            assert lo + tb <= plan.row_off[b["expert"][s] + 1]
        assert 1 <= v <= tb

    # minimal padding, bound per X_e and per rank
    total_pad = 0
    for e in range(plan.E_l):
        pad_e = 0
        for o in range(W):
            c = int(plan.c[e, o])
            if o == r:
                continue
            p = (-(-c // tb) * tb) - c
            assert 0 <= p < tb
            pad_e += p
        real = int(np.count_nonzero(src[plan.row_off[e]:plan.row_off[e + 1]] >= 0))
        assert plan.m_e[e] - real == pad_e
        assert pad_e <= padding_bound(W, tb), f"expert {e}: padding {pad_e} over the bound"
        total_pad += pad_e
    assert total_pad <= plan.E_l * padding_bound(W, tb)
    assert int(np.count_nonzero(src < 0)) == total_pad

    # schedule rules
    remote = b["remote"].astype(bool)
    assert np.all(remote[:plan.n_remote]) and not np.any(remote[plan.n_remote:])
    seq = [int(e) for i, e in enumerate(b["expert"][:plan.n_remote])
           if i == 0 or e != b["expert"][i - 1]]
    assert len(seq) == len(set(seq)), "remote bands of one expert are not contiguous"
    counts = [int(plan.rb[e]) for e in seq]
    assert counts == sorted(counts, reverse=True), "rule (ii) violated"

    # combine plan: disjoint intervals, exact group coverage, no padding sent
    for o in range(W):
        sel = np.nonzero(b["dst"] == o)[0]
        iv = sorted((int(b["dst_off"][s]), int(b["dst_off"][s] + b["valid"][s])) for s in sel)
        for (a0, a1), (b0, b1) in zip(iv, iv[1:]):
            assert a1 <= b0, f"owner {o}: overlapping writes"
        for e in range(plan.E_l):
            se = sel[b["expert"][sel] == e]
            assert int(b["valid"][se].sum()) == int(plan.c[e, o])
    sent = np.zeros(plan.M, dtype=np.int64)
    for s in range(B):
        sent[int(b["src_row"][s]):int(b["src_row"][s] + b["valid"][s])] += 1
    assert np.all(sent[src < 0] == 0), "a padding row is sent"
    assert np.all(sent[src >= 0] == 1), "a real row is not sent exactly once"

    # segments
    sg = plan.segs
    nrs = plan.n_remote_segs
    covered = []
    for q in range(sg["first_band"].shape[0]):
        f0, nb = int(sg["first_band"][q]), int(sg["n_bands"][q])
        run = list(range(f0, f0 + nb))
        covered += run
        assert nb <= max(plan.mgb, 1)
        keys = {(int(b["expert"][s]), int(b["dst"][s])) for s in run}
        assert len(keys) == 1, "segment crosses a group"
        rows = 0
        for s in run:
            assert int(b["src_row"][s]) == int(sg["src_row"][q]) + rows
            assert int(b["dst_off"][s]) == int(sg["dst_off"][q]) + rows
            rows += int(b["valid"][s])
        assert rows == int(sg["rows"][q])
    assert covered == list(range(B)), "segments do not tile the band list in order"
    if plan.n_remote >= 1:
        assert int(sg["n_bands"][0]) == 1
        assert int(sg["first_band"][nrs - 1] + sg["n_bands"][nrs - 1]) == plan.n_remote
        assert int(sg["n_bands"][nrs - 1]) == 1
