"""Combine (test infrastructure only): the second all-to-all of the tile-signal
notes (§2.2 step 4) driven by the combine plan of §4.5.  Every band sends its
``valid`` rows, starting at layout row ``src_row``, to owner ``dst`` at row
``dst_off``; padding rows are never sent."""
from __future__ import annotations

import numpy as np


def layout_x(plan, x_recv_bits: np.ndarray) -> np.ndarray:
    """The owner-aligned layout X [M, d] (notes §4.2): received row
    src_index[row], or zeros for a padding row."""
    d = x_recv_bits.shape[1]
    X = np.zeros((plan.M, d), dtype=np.uint16)
    real = plan.src_index >= 0
    X[real] = x_recv_bits[plan.src_index[real]]
    return X


def apply(plan, y_bits: np.ndarray, recv: list) -> list:
    """Write the expert output rows into the owners' receive buffers (copies
    of ``recv`` are modified and returned)."""
    out = [np.array(p, copy=True) for p in recv]
    b = plan.bands
    for s in range(b["expert"].shape[0]):
        n = int(b["valid"][s])
        src = int(b["src_row"][s])
        dst = int(b["dst"][s])
        off = int(b["dst_off"][s])
        out[dst][off:off + n] = y_bits[src:src + n]
    return out


def written_rows(plan) -> dict:
    """For every owner, the receive-buffer rows this rank writes and the layout
    row each comes from."""
    res = {o: ([], []) for o in range(plan.W)}
    b = plan.bands
    for s in range(b["expert"].shape[0]):
        n = int(b["valid"][s])
        res[int(b["dst"][s])][0].extend(range(int(b["dst_off"][s]), int(b["dst_off"][s]) + n))
        res[int(b["dst"][s])][1].extend(range(int(b["src_row"][s]), int(b["src_row"][s]) + n))
    return {o: (np.array(a, dtype=np.int64), np.array(c, dtype=np.int64)) for o, (a, c) in res.items()}
