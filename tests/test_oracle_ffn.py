"""Pins for the oracle's SwiGLU expert FFN and scale (CPU only).

* Closed-form fixtures (tests/golden/ffn_closed_form.json): a scalar case
  and a permutation case that fails on swapped gate/up, a transposed weight
  or a wrong bf16 rounding point.
* silu identities: silu(0) = 0, silu(-z) = silu(z) - z, silu(ln 3) = 0.75 ln 3,
  and agreement with torch's silu (library routine) in float64.
* Zero (padding) rows give exactly zero output.
* Scale special cases: k = 1 with weight 1 returns the row; identical rows
  give (sum of weights) * row.
"""
import json
import math
import os

import numpy as np
import torch

from oracle import bf16, ffn, scale

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "ffn_closed_form.json")) as fh:
        return json.load(fh)


def _bits(a):
    return bf16.to_bits(np.asarray(a, dtype=np.float64))


def test_scalar_closed_form():
    g = _gold()["scalar"]
    x = _bits([[g["x"]]])
    wgu = _bits([[g["w_gate"]], [g["w_up"]]])
    wd = _bits([[g["w_down"]]])
    h, y = ffn.expert_rows(x, wgu, wd)
    assert bf16.from_bits(h)[0, 0] == g["h"]
    assert bf16.from_bits(y)[0, 0] == g["y"]


def test_permutation_closed_form():
    g = _gold()["permutation"]
    n = len(g["x"])
    def pick(p):
        m = np.zeros((n, n))
        m[np.arange(n), p] = 1.0
        return m
    x = _bits([g["x"]])
    wgu = _bits(np.concatenate([pick(g["gate_pick"]), pick(g["up_pick"])]))
    wd = _bits(pick(g["down_pick"]))
    h, y = ffn.expert_rows(x, wgu, wd)
    assert bf16.from_bits(h)[0].tolist() == g["h"]
    assert bf16.from_bits(y)[0].tolist() == g["y"]


def test_silu_identities():
    z = np.linspace(-20, 20, 4001)
    s = ffn.silu(z)
    assert ffn.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(ffn.silu(-z), s - z, rtol=0, atol=1e-12)
    assert abs(ffn.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(s, ref, rtol=1e-14, atol=1e-14)


def test_zero_rows_give_zero():
    rng = np.random.default_rng(0)
    wgu = _bits(rng.standard_normal((64, 32)) * 0.1)
    wd = _bits(rng.standard_normal((32, 32)) * 0.1)
    h, y = ffn.expert_rows(np.zeros((3, 32), np.uint16), wgu, wd)
    assert np.all(bf16.from_bits(h) == 0) and np.all(bf16.from_bits(y) == 0)


def test_scale_special_cases():
    rng = np.random.default_rng(1)
    rows = _bits(rng.standard_normal((6, 16)))
    # k = 1, weight 1: output is the row itself
    out = scale.scale(rows, np.ones((6, 1), np.float32), np.arange(6).reshape(6, 1))
    assert np.array_equal(out, rows)
    # identical rows: (sum of weights) * row, weights exact in binary
    same = np.repeat(rows[:1], 3, axis=0)
    w = np.array([[0.5, 0.25, 0.125]], np.float32)
    out = scale.scale(same, w, np.array([[0, 1, 2]]))
    assert np.array_equal(out[0], _bits(0.875 * bf16.from_bits(rows[0])))
    # slot order through pos: permuted rows with permuted pos give the same
    w2 = np.array([[0.5, 0.25]], np.float32)
    a = scale.scale(rows[:2], w2, np.array([[0, 1]]))
    b = scale.scale(rows[1::-1].copy(), w2, np.array([[1, 0]]))
    assert np.array_equal(a, b)
