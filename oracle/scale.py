"""Scale (test infrastructure only): the gate-weighted reduction at the owner
(tile-signal notes §2.2 step 5, §2.1: the layer output is the gate-weighted sum
of the k selected experts' outputs).  Token t's output is the sum over its k
slots of weight * returned row, in float64, rounded once to bf16."""
from __future__ import annotations

import numpy as np

from . import bf16


def scale(recv_bits: np.ndarray, topk_w: np.ndarray, pos: np.ndarray, tokens=None) -> np.ndarray:
    """out[t] = bf16(sum_j w[t, j] * recv[pos[t, j]]) for the given tokens
    (all by default).  recv_bits [T*k, d] bf16 bits, topk_w [T, k], pos [T, k]."""
    if tokens is None:
        tokens = np.arange(pos.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)[tokens]           # [n, k]
    rows = bf16.from_bits(recv_bits[pos[tokens]])               # [n, k, d]
    acc = np.einsum("nk,nkd->nd", w, rows)
    return bf16.to_bits(acc)
