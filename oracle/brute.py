"""Definition-level references for tiny inputs (test infrastructure only).

``moe_output``: the MoE layer output straight from its definition (tile-signal
notes §2.1: the output is the gate-weighted sum of the top-k experts' FFN
outputs; §2.2 five-step forward), token by token and slot by slot, without any
layout, band or plan.  The two bf16 rounding points of the expert FFN (hidden
activation, expert output) and the final rounding of the sum are the same as
in the method, so for a correct plan the method's per-token result is equal to
this one.

``layout_by_sorting``: the owner-aligned layout of notes §4.2 obtained by
sorting the received rows with the key (expert, position of the owner in the
remote-first owner order, arrival index) and inserting padding after each
remote group; no histogram, scan or offset arithmetic is involved.
"""
from __future__ import annotations

import numpy as np

from . import bf16
from .ffn import silu


def expert_ffn_row(x_bits, w_gate_up_bits, w_down_bits):
    x = bf16.from_bits(x_bits)
    wgu = bf16.from_bits(w_gate_up_bits)
    f = wgu.shape[0] // 2
    gate = wgu[:f] @ x
    up = wgu[f:] @ x
    h = bf16.round_f64(silu(gate) * up)
    return bf16.round_f64(bf16.from_bits(w_down_bits) @ h)


def moe_output(x_owner_bits, topk_ids, topk_w, weight_of):
    """out [N, d] bf16 bits.  ``weight_of(g)`` returns (w_gate_up [2f, d],
    w_down [d, f]) bf16 bits of global expert g."""
    N, k = topk_ids.shape
    cache = {}
    out = np.empty_like(x_owner_bits)
    for n in range(N):
        acc = np.zeros(x_owner_bits.shape[1], dtype=np.float64)
        for j in range(k):
            g = int(topk_ids[n, j])
            if g not in cache:
                cache[g] = weight_of(g)
            wgu, wd = cache[g]
            acc += float(topk_w[n, j]) * expert_ffn_row(x_owner_bits[n], wgu, wd)
        out[n] = bf16.to_bits(acc)
    return out


def layout_by_sorting(topk_ids, tokens, r, E_l, tb_m):
    """List of layout entries per local expert: received row index or -1."""
    W = len(tokens)
    k = topk_ids.shape[1]
    order_pos = {o: p for p, o in enumerate([o for o in range(W) if o != r] + [r])}
    items = []
    i = 0
    n0 = 0
    for o in range(W):
        for t in range(tokens[o]):
            for j in range(k):
                g = int(topk_ids[n0 + t, j])
                if r * E_l <= g < (r + 1) * E_l:
                    items.append((g - r * E_l, order_pos[o], i, o))
                    i += 1
        n0 += tokens[o]
    items.sort()
    layout = {e: [] for e in range(E_l)}
    for idx, (e, p, i, o) in enumerate(items):
        layout[e].append(i)
        last_of_group = idx + 1 == len(items) or items[idx + 1][:2] != (e, p)
        if last_of_group and o != r:
            count = sum(1 for it in items if it[0] == e and it[1] == p)
            while count % tb_m:
                layout[e].append(-1)
                count += 1
    return layout
