"""The seeded input generator (CPU only): determinism, shapes, the routing
recipe and the dispatch order the boundary expects."""
import numpy as np

import synth
from oracle import plan as P


def test_owner_skew_counts():
    assert synth.owner_token_counts(8, 1024, skew=4.0) == (1638,) * 4 + (410,) * 4
    assert synth.get_config("dsv3_skew").N == 8192


def test_routing_shapes_and_weights():
    for name in ["tiny", "qwen3", "dsv3_skew", "decode_tb32"]:
        cfg = synth.get_config(name)
        ids, w = synth.routing(cfg)
        assert ids.shape == (cfg.N, cfg.k) and ids.dtype == np.int32
        assert ids.min() >= 0 and ids.max() < cfg.E
        srt = np.sort(ids, axis=1)
        assert np.all(srt[:, 1:] != srt[:, :-1])          # k distinct experts
        if cfg.weights == "renorm":
            assert np.allclose(w.sum(axis=1), 1.0, atol=1e-5)
        else:
            assert np.all(w.sum(axis=1) <= 1.0 + 1e-6)
        ids2, w2 = synth.routing(cfg)
        assert np.array_equal(ids, ids2) and np.array_equal(w, w2)


def test_zipf_puts_hot_experts_on_rank0():
    cfg = synth.get_config("dsv3_skew")
    ids, _ = synth.routing(cfg)
    per_rank = np.bincount(ids.reshape(-1) // cfg.E_l, minlength=cfg.W)
    assert per_rank[0] == per_rank.max()


def test_dispatch_order_matches_oracle_enumeration():
    cfg = synth.get_config("tiny")
    ids, _ = synth.routing(cfg)
    x = synth.activations(cfg)
    x_recv, tok = synth.dispatch(cfg, ids, x)
    o, t, j, e = P.received_rows(ids, cfg.tokens, cfg.rank, cfg.E_l)
    off = P.owner_offsets(cfg.tokens)
    assert np.array_equal(tok, off[o] + t)
    assert np.array_equal(x_recv, x[off[o] + t])


def test_weights_are_deterministic_bf16():
    cfg = synth.get_config("tiny")
    a1, b1 = synth.expert_weights(cfg, 3)
    a2, b2 = synth.expert_weights(cfg, 3)
    assert a1.shape == (2 * cfg.f, cfg.d) and b1.shape == (cfg.d, cfg.f)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
    v = synth.bits_to_float(a1)
    assert 0.015 < float(v.std()) < 0.025
