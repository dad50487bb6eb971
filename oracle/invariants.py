"""Properties the pages fix for layout, schedule and combine plan (test
infrastructure only).

``check(plan)`` evaluates every property below on its own and raises one
AssertionError that names every violated property (``violations(plan)``
returns the names without raising).  Each property is computed from the
plan's arrays, never from the formula that built them, so that a builder
mistake shows up as a named violation:

* tile-signal notes §4.2: every band holds rows of exactly one owner and one
  expert (``mixed-owners``, ``wrong-expert``); its valid rows are real rows
  (``padding-inside-valid``) and, for a remote band, the rest of its tb_M
  rows are padding (``remote-tail-not-padding``); 1 <= valid <= tb_M
  (``band-valid-range``);
* §4.2 / §4.4 (the pseudo-code pads only remote groups): the groups of X_e
  come in ascending owner rank with the local rank last (``group-order``);
  the local group is not padded (``local-group-padded``); every
  remote group is followed by exactly the padding that reaches the next
  multiple of tb_M (``padding-not-minimal``);
* §4.3 / §4.5: the padding rows counted in X_e are at most (W-1)(tb_M-1)
  (``padding-bound-expert``), and at most E_l times that for the rank
  (``padding-bound-rank``);
* §4.4 rule (i): every remote band precedes every local band
  (``remote-after-local``); rule (ii): the remote bands of one expert are
  consecutive (``remote-bands-not-contiguous``) and the experts appear in
  non-increasing order of remote band count (``rule-ii``);
* §4.5: the write intervals of one rank's plan are disjoint within every
  owner's receive buffer (``overlapping-writes``) and cover exactly the
  group's rows (``group-coverage``); padding rows are never sent
  (``padding-sent``) and every real row is sent exactly once
  (``row-not-sent-once``);
* §5.2: segments tile the band list in order (``segments-do-not-tile``),
  hold at most mgb bands (``segment-too-long``), never cross a group
  (``segment-crosses-group``), are contiguous at both ends
  (``segment-not-contiguous``) with the right row count
  (``segment-rows``); the first and the last remote segment are single bands
  (``first-segment``, ``last-segment``).
"""
from __future__ import annotations

from typing import List

import numpy as np

from .plan import padding_bound


def violations(plan) -> List[str]:
    """Names of every violated property (empty for a valid plan)."""
    bad = set()
    W, r, tb = plan.W, plan.r, plan.tb_m
    b = plan.bands
    B = plan.n_bands
    src = np.asarray(plan.src_index)
    M = src.shape[0]
    row_off = np.asarray(plan.row_off)

    # --- bands: one owner, one expert, padding only in remote band tails ---
    for s in range(B):
        lo = int(b["src_row"][s])
        v = int(b["valid"][s])
        if not 1 <= v <= tb:
            bad.add("band-valid-range")
        rows = src[lo:lo + max(v, 0)]
        if np.any(rows < 0):
            bad.add("padding-inside-valid")
        real = rows[rows >= 0]
        if np.any(plan.recv_owner[real] != b["dst"][s]):
            bad.add("mixed-owners")
        if np.any(plan.recv_expert[real] != b["expert"][s]):
            bad.add("wrong-expert")
        if b["remote"][s] and np.any(src[lo + v:lo + tb] != -1):
            bad.add("remote-tail-not-padding")

    # --- layout of every X_e, read off src_index ---
    total_pad = 0
    for e in range(plan.E_l):
        a, z = int(row_off[e]), int(row_off[e + 1])
        seg = src[a:z]
        pad_e = int(np.count_nonzero(seg < 0))
        total_pad += pad_e
        if pad_e > padding_bound(W, tb):
            bad.add("padding-bound-expert")
        # walk X_e: runs of one owner's rows, each followed by its padding
        i = 0
        n = seg.shape[0]
        seen_local = False
        seq_o = []
        while i < n:
            if seg[i] < 0:
                # padding with no group before it in this X_e
                bad.add("padding-not-minimal")
                while i < n and seg[i] < 0:
                    i += 1
                continue
            o = int(plan.recv_owner[seg[i]])
            seq_o.append(o)
            j = i
            while j < n and seg[j] >= 0 and int(plan.recv_owner[seg[j]]) == o:
                j += 1
            c = j - i
            p = 0
            while j + p < n and seg[j + p] < 0:
                p += 1
            if o == r:
                seen_local = True
                if p != 0 or j + p != n:
                    bad.add("local-group-padded")
            else:
                if seen_local:
                    bad.add("group-order")
                if p != (-c) % tb:
                    bad.add("padding-not-minimal")
            i = j + p
        remote_seq = [o for o in seq_o if o != r]
        if remote_seq != sorted(set(remote_seq)) or (r in seq_o and seq_o[-1] != r):
            bad.add("group-order")
    if total_pad > plan.E_l * padding_bound(W, tb):
        bad.add("padding-bound-rank")
    if int(np.count_nonzero(src < 0)) != total_pad:
        bad.add("padding-not-minimal")

    # --- schedule rules ---
    remote = b["remote"].astype(bool)
    nr = int(plan.n_remote)
    if not (np.all(remote[:nr]) and not np.any(remote[nr:])):
        bad.add("remote-after-local")
    first_local = np.nonzero(~remote)[0]
    if first_local.size and np.any(remote[first_local[0]:]):
        bad.add("remote-after-local")
    rem_idx = np.nonzero(remote)[0]
    seq = [int(b["expert"][s]) for i, s in enumerate(rem_idx)
           if i == 0 or b["expert"][s] != b["expert"][rem_idx[i - 1]]]
    if len(seq) != len(set(seq)):
        bad.add("remote-bands-not-contiguous")
    counts = [int(np.count_nonzero(b["expert"][rem_idx] == e)) for e in seq]
    if counts != sorted(counts, reverse=True):
        bad.add("rule-ii")

    # --- combine plan ---
    for o in range(W):
        sel = np.nonzero(b["dst"] == o)[0]
        iv = sorted((int(b["dst_off"][s]), int(b["dst_off"][s] + b["valid"][s])) for s in sel)
        for (a0, a1), (b0, b1) in zip(iv, iv[1:]):
            if a1 > b0:
                bad.add("overlapping-writes")
        for e in range(plan.E_l):
            se = sel[b["expert"][sel] == e]
            if int(b["valid"][se].sum()) != int(plan.c[e, o]):
                bad.add("group-coverage")
    sent = np.zeros(M, dtype=np.int64)
    for s in range(B):
        lo = int(b["src_row"][s])
        sent[lo:lo + int(b["valid"][s])] += 1
    if np.any(sent[src < 0] != 0):
        bad.add("padding-sent")
    if np.any(sent[src >= 0] != 1):
        bad.add("row-not-sent-once")

    # --- segments ---
    sg = plan.segs
    nrs = int(plan.n_remote_segs)
    covered = []
    for q in range(sg["first_band"].shape[0]):
        f0, nb = int(sg["first_band"][q]), int(sg["n_bands"][q])
        run = list(range(f0, f0 + nb))
        covered += run
        if nb > max(plan.mgb, 1):
            bad.add("segment-too-long")
        run_in = [s for s in run if 0 <= s < B]
        keys = {(int(b["expert"][s]), int(b["dst"][s])) for s in run_in}
        if len(keys) > 1:
            bad.add("segment-crosses-group")
        rows = 0
        for s in run_in:
            if (int(b["src_row"][s]) != int(sg["src_row"][q]) + rows or
                    int(b["dst_off"][s]) != int(sg["dst_off"][q]) + rows):
                bad.add("segment-not-contiguous")
            rows += int(b["valid"][s])
        if rows != int(sg["rows"][q]):
            bad.add("segment-rows")
    if covered != list(range(B)):
        bad.add("segments-do-not-tile")
    if nr >= 1 and nrs >= 1:
        if int(sg["n_bands"][0]) != 1:
            bad.add("first-segment")
        if int(sg["n_bands"][nrs - 1]) != 1 or \
                int(sg["first_band"][nrs - 1] + sg["n_bands"][nrs - 1]) != nr:
            bad.add("last-segment")
    return sorted(bad)


def check(plan, topk_ids=None) -> None:
    """Raise AssertionError naming every violated property."""
    v = violations(plan)
    assert not v, "plan violates: " + ", ".join(v)
