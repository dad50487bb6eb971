"""The oracle's method path against the definition of the MoE layer (CPU only).

For every rank r of a small layer, the oracle's plan, owner-aligned layout,
FFN on the layout (padding rows included) and combine are run into shared
owner receive buffers; then every owner scales its tokens.  The result must
equal, element for element, the MoE output computed token by token from its
definition (oracle.brute.moe_output: gate-weighted sum of the top-k experts'
FFN outputs), which involves no layout, band, plan or slot table.  This pins
the whole chain (received-row order, grouping, padding, bands, offsets, slot
table, FFN wiring, scale) on the named tiny workload and on random shapes.
"""
import numpy as np
import pytest

import synth
from oracle import brute, combine, ffn, plan as P, scale


def _run_all_ranks(cfg, ids, w, x_owner, weight_of):
    W, E_l, k = cfg.W, cfg.E_l, cfg.k
    off = P.owner_offsets(cfg.tokens)
    recv = [np.zeros((cfg.tokens[o] * k, cfg.d), np.uint16) for o in range(W)]
    for r in range(W):
        pl = P.build_plan(ids, cfg.tokens, r, E_l, cfg.tb_m, cfg.mgb)
        x_recv, _ = synth.dispatch(cfg, ids, x_owner, rank=r)
        X = combine.layout_x(pl, x_recv)
        wgu = np.stack([weight_of(r * E_l + e)[0] for e in range(E_l)])
        wd = np.stack([weight_of(r * E_l + e)[1] for e in range(E_l)])
        _, Y = ffn.layout_rows(pl, X, wgu, wd, np.arange(pl.M))
        assert np.all(Y[pl.src_index < 0] == 0) if pl.M else True
        recv = combine.apply(pl, Y, recv)
    out = np.empty((cfg.N, cfg.d), np.uint16)
    for o in range(W):
        pl_o = P.build_plan(ids, cfg.tokens, o, E_l, cfg.tb_m, cfg.mgb)
        out[off[o]:off[o + 1]] = scale.scale(recv[o], w[off[o]:off[o + 1]], pl_o.pos)
    return out


@pytest.mark.parametrize("name", ["tiny", "tiny_unit"])
def test_named_tiny_layer_equals_definition(name):
    cfg = synth.get_config(name)
    ids, w = synth.routing(cfg)
    x = synth.activations(cfg)
    cache = {}
    def weight_of(g):
        if g not in cache:
            cache[g] = synth.expert_weights(cfg, g)
        return cache[g]
    got = _run_all_ranks(cfg, ids, w, x, weight_of)
    ref = brute.moe_output(x, ids, w, weight_of)
    assert np.array_equal(got, ref)


def test_random_small_layers_equal_definition():
    rng = np.random.default_rng(7)
    for trial in range(6):
        W = int(rng.integers(1, 5))
        E_l = int(rng.integers(1, 3))
        k = int(rng.integers(1, min(W * E_l, 3) + 1))
        tokens = tuple(int(rng.integers(0, 9)) for _ in range(W))
        cfg = synth.MoEConfig("rand", W, W * E_l, tokens, 16, 8, k, int(rng.choice([1, 2, 4])),
                              seed=100 + trial, mgb=int(rng.integers(1, 3)))
        ids = synth.random_routing_case(rng, W, E_l, k, list(tokens))
        w = rng.random((cfg.N, k)).astype(np.float32)
        x = synth.activations(cfg)
        weight_of = lambda g, cfg=cfg: synth.expert_weights(cfg, g)
        got = _run_all_ranks(cfg, ids, w, x, weight_of)
        ref = brute.moe_output(x, ids, w, weight_of)
        assert np.array_equal(got, ref), trial
