"""Layout, schedule and combine plan of one rank (test infrastructure only).

Follows the tile-signal notes:

* §4.2 / layout half of the §4.4 pseudo-code: for every local expert e, the
  received rows are grouped by owner rank; every *remote* group is zero-padded
  up to a multiple of tb_M; the groups are concatenated with the remote owners
  first (ascending rank, the local rank skipped) and the local group last.
* §4.4 / schedule half of the pseudo-code: rule (ii) orders the local experts
  by their number of remote row bands, descending; rule (i) puts every remote
  band of every expert before any local band.
* §4.5: the combine plan gives each band its destination rank, its write
  offset in that rank's receive buffer and its count of valid (non-pad) rows;
  offsets are coordinated across local experts so they never overlap.
* §5.2: bands are merged into segments; the first and the last segment hold
  one band, the middle ones up to ``mgb`` bands.

Readings taken where the pages leave a step open (each is listed in the
design notes of the repository):

* arrival order of received rows is (owner, token, slot) lexicographic and a
  group keeps that order (stable);
* the local group is not padded (the pseudo-code pads only remote groups and
  the padding bound counts W-1 groups);
* an empty group contributes no rows and no bands;
* ties in rule (ii) go to the lower local expert id; local bands follow in
  ascending expert id;
* owner o's receive buffer holds its T_o*k returned rows ordered by (global
  expert, token), so the band of group (e, o) with index b starts at
  base_o(g) + b*tb_M where base_o(g) counts owner o's (token, slot) pairs
  whose expert id is below g = r*E_l + e;
* local bands are part of the plan too (destination = the rank itself) and
  are copied after the remote ones;
* segments never cross a (expert, destination) group; the first/last rule
  applies to the remote prefix; local segments are greedy runs of <= mgb
  bands of one expert.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np


@dataclasses.dataclass
class Plan:
    W: int
    r: int
    E_l: int
    tb_m: int
    mgb: int
    tokens: tuple
    # received rows, in arrival order i = 0..R-1
    recv_owner: np.ndarray
    recv_token: np.ndarray      # token index within its owner
    recv_slot: np.ndarray
    recv_expert: np.ndarray     # local expert id
    # layout
    c: np.ndarray               # [E_l, W] rows of local expert e from owner o
    grp_off: np.ndarray         # [E_l, W] start of group (e, o) inside X_e
    m_e: np.ndarray             # [E_l] rows of X_e (padding included)
    row_off: np.ndarray         # [E_l + 1] start of X_e in the layout
    src_index: np.ndarray       # [M] received row index, -1 for padding
    base: np.ndarray            # [W, E_l] base_o(r*E_l + e)
    # schedule: bands in S order
    bands: Dict[str, np.ndarray]
    n_remote: int
    rb: np.ndarray              # [E_l] remote bands per expert
    expert_order: np.ndarray    # [E_l] rule (ii) order
    segs: Dict[str, np.ndarray]
    n_remote_segs: int
    pos: np.ndarray             # [T_r, k] owner-side slot of (token, slot)

    @property
    def R(self) -> int:
        return int(self.recv_owner.shape[0])

    @property
    def M(self) -> int:
        return int(self.row_off[-1])

    @property
    def n_bands(self) -> int:
        return int(self.bands["expert"].shape[0])


def owner_offsets(tokens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(tokens, dtype=np.int64))])


def received_rows(topk_ids: np.ndarray, tokens, r: int, E_l: int):
    """(owner, token, slot, local expert) of every received row, in arrival
    order: all (o, t, j) triples whose expert lives on rank r, enumerated
    lexicographically."""
    W = len(tokens)
    k = topk_ids.shape[1]
    off = owner_offsets(tokens)
    o_l, t_l, j_l, e_l = [], [], [], []
    for o in range(W):
        block = topk_ids[off[o]:off[o + 1]]          # [T_o, k]
        g = block.reshape(-1)
        local = np.nonzero((g >= r * E_l) & (g < (r + 1) * E_l))[0]
        o_l.append(np.full(local.shape, o, dtype=np.int64))
        t_l.append(local // k)
        j_l.append(local % k)
        e_l.append(g[local].astype(np.int64) - r * E_l)
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)
    return cat(o_l), cat(t_l), cat(j_l), cat(e_l)


def owner_order(W: int, r: int) -> List[int]:
    """Remote owners in ascending rank, then the local rank last."""
    return [o for o in range(W) if o != r] + [r]


def padded(c: int, tb_m: int) -> int:
    """Rows a remote group of c rows occupies: the next multiple of tb_M."""
    return -(-c // tb_m) * tb_m


def build_plan(topk_ids: np.ndarray, tokens, r: int, E_l: int, tb_m: int,
               mgb: int = 1) -> Plan:
    topk_ids = np.asarray(topk_ids)
    W = len(tokens)
    k = topk_ids.shape[1]
    off = owner_offsets(tokens)
    ro, rt, rj, re = received_rows(topk_ids, tokens, r, E_l)

    # --- owner-aligned layout (notes §4.2, layout half of the §4.4 code) ---
    c = np.zeros((E_l, W), dtype=np.int64)
    for e, o in zip(re, ro):
        c[e, o] += 1
    grp_off = np.zeros((E_l, W), dtype=np.int64)
    m_e = np.zeros(E_l, dtype=np.int64)
    for e in range(E_l):
        running = 0
        for o in owner_order(W, r):
            grp_off[e, o] = running
            running += padded(int(c[e, o]), tb_m) if o != r else int(c[e, o])
        m_e[e] = running
    row_off = np.concatenate([[0], np.cumsum(m_e)]).astype(np.int64)
    M = int(row_off[-1])
    src_index = np.full(M, -1, dtype=np.int64)
    for e in range(E_l):
        for o in range(W):
            members = np.nonzero((re == e) & (ro == o))[0]    # ascending i
            start = row_off[e] + grp_off[e, o]
            src_index[start:start + members.shape[0]] = members

    # --- receive-buffer bases (notes §4.5): owner o's pairs below expert g ---
    base = np.zeros((W, E_l), dtype=np.int64)
    for o in range(W):
        ids_o = topk_ids[off[o]:off[o + 1]]
        for e in range(E_l):
            base[o, e] = int(np.count_nonzero(ids_o < r * E_l + e))

    # --- row bands of each X_e, in X_e order ---
    per_expert: List[List[dict]] = []
    for e in range(E_l):
        lst = []
        for o in owner_order(W, r):
            n = int(c[e, o])
            for b in range(-(-n // tb_m)):
                lst.append(dict(expert=e, dst=o, b=b,
                                src_row=int(row_off[e] + grp_off[e, o] + b * tb_m),
                                dst_off=int(base[o, e] + b * tb_m),
                                valid=min(tb_m, n - b * tb_m),
                                remote=int(o != r)))
        per_expert.append(lst)

    # --- remote-first schedule (notes §4.4, rules (i) and (ii)) ---
    rb = np.array([sum(x["remote"] for x in per_expert[e]) for e in range(E_l)],
                  dtype=np.int64)
    expert_order = np.array(sorted(range(E_l), key=lambda e: (-rb[e], e)), dtype=np.int64)
    S = []
    for e in expert_order:
        S += [x for x in per_expert[e] if x["remote"]]
    n_remote = len(S)
    for e in range(E_l):
        S += [x for x in per_expert[e] if not x["remote"]]
    fields = ["expert", "dst", "b", "src_row", "dst_off", "valid", "remote"]
    bands = {f: np.array([x[f] for x in S], dtype=np.int64) for f in fields}

    segs, n_remote_segs = build_segments(bands, n_remote, mgb)

    # --- owner-side slots of the simulated rank's own tokens ---
    ids_r = topk_ids[off[r]:off[r + 1]].reshape(-1)
    order = np.argsort(ids_r, kind="stable")          # (expert, token) order
    pos = np.empty(ids_r.shape[0], dtype=np.int64)
    pos[order] = np.arange(ids_r.shape[0])
    pos = pos.reshape(-1, k)

    return Plan(W=W, r=r, E_l=E_l, tb_m=tb_m, mgb=mgb, tokens=tuple(int(x) for x in tokens),
                recv_owner=ro, recv_token=rt, recv_slot=rj, recv_expert=re,
                c=c, grp_off=grp_off, m_e=m_e, row_off=row_off, src_index=src_index,
                base=base, bands=bands, n_remote=n_remote, rb=rb,
                expert_order=expert_order, segs=segs, n_remote_segs=n_remote_segs, pos=pos)


def build_segments(bands: Dict[str, np.ndarray], n_remote: int, mgb: int):
    """Segments over the band list S (notes §5.2): the first remote band alone,
    the last remote band alone, greedy runs of <= mgb bands of one
    (expert, destination) group in between; local bands in greedy runs of
    <= mgb bands of one expert."""
    B = bands["expert"].shape[0]
    runs: List[List[int]] = []

    def group(s):
        return (int(bands["expert"][s]), int(bands["dst"][s]))

    def greedy(lo, hi):
        cur: List[int] = []
        for s in range(lo, hi):
            if cur and (len(cur) == mgb or group(s) != group(cur[-1])):
                runs.append(cur)
                cur = []
            cur.append(s)
        if cur:
            runs.append(cur)

    if n_remote >= 1:
        runs.append([0])
    if n_remote >= 3:
        greedy(1, n_remote - 1)
    if n_remote >= 2:
        runs.append([n_remote - 1])
    n_remote_segs = len(runs)
    greedy(n_remote, B)

    out = {k: [] for k in ["first_band", "n_bands", "dst", "dst_off", "src_row", "rows"]}
    for run in runs:
        s0 = run[0]
        out["first_band"].append(s0)
        out["n_bands"].append(len(run))
        out["dst"].append(int(bands["dst"][s0]))
        out["dst_off"].append(int(bands["dst_off"][s0]))
        out["src_row"].append(int(bands["src_row"][s0]))
        out["rows"].append(int(sum(int(bands["valid"][s]) for s in run)))
    return {k: np.array(v, dtype=np.int64) for k, v in out.items()}, n_remote_segs


def padding_bound(W: int, tb_m: int) -> int:
    """Worst-case padding of one X_e (notes §4.3 and §4.5): W-1 padded groups,
    each short of a multiple of tb_M by at most tb_M - 1 rows."""
    return (W - 1) * (tb_m - 1)
