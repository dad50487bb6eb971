"""SwiGLU expert FFN (test infrastructure only).

The tile-signal notes describe expert computation as GEMM, activation, GEMM
(§2.2 step 3, §2.3); the workload fixes the activation as SwiGLU:
``y = W_down (silu(W_gate x) * (W_up x))`` with ``silu(z) = z / (1 + e^-z)``,
no biases.  Arithmetic is float64; the hidden activation h and the expert
output y are each rounded once to bf16 (the two tensors the path stores).
The notes' zero-padded rows (§4.2 step 2) go through the same arithmetic and
come out as zeros.
"""
from __future__ import annotations

import numpy as np

from . import bf16


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_rows(x_bits: np.ndarray, w_gate_up_bits: np.ndarray, w_down_bits: np.ndarray):
    """FFN of one expert on rows x [n, d] (bf16 bits).  w_gate_up [2f, d] holds
    the gate projection in rows 0..f-1 and the up projection in rows f..2f-1;
    w_down is [d, f].  Returns (h bits [n, f], y bits [n, d])."""
    x = bf16.from_bits(x_bits)
    wgu = bf16.from_bits(w_gate_up_bits)
    f = wgu.shape[0] // 2
    gate = x @ wgu[:f].T
    up = x @ wgu[f:].T
    h_bits = bf16.to_bits(silu(gate) * up)
    y = bf16.from_bits(h_bits) @ bf16.from_bits(w_down_bits).T
    return h_bits, bf16.to_bits(y)


def layout_rows(plan, x_layout_bits, w_gate_up_bits, w_down_bits, rows):
    """FFN of the given layout rows (each row uses the weights of the expert
    whose X_e contains it).  Returns (h bits [len(rows), f], y bits)."""
    rows = np.asarray(rows, dtype=np.int64)
    expert = np.searchsorted(plan.row_off, rows, side="right") - 1
    f = w_gate_up_bits.shape[1] // 2
    d = w_down_bits.shape[1]
    h = np.empty((rows.shape[0], f), dtype=np.uint16)
    y = np.empty((rows.shape[0], d), dtype=np.uint16)
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        hh, yy = expert_rows(x_layout_bits[rows[sel]], w_gate_up_bits[e], w_down_bits[e])
        h[sel] = hh
        y[sel] = yy
    return h, y
