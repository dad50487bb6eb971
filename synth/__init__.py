"""Seeded synthetic inputs for one expert-parallel rank's share of an MoE layer.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It holds none of the method's arithmetic: it only draws routing,
activations and expert weights, stores them as bf16 bit patterns, and performs
the token dispatch that precedes the method (step 2 of the five-step MoE
forward in the tile-signal reading notes, "MoE 计算-通信细粒度重叠：用 Tile 级信号把
All-to-All 藏在 GEMM 背后", §2.2), which the method takes as its input.

Workloads (all seed 0, rank 0 simulated):

==============  ==  ====  ===========  ====  =====  =  ===========================
name            W   E     T per owner  d     f      k  routing
==============  ==  ====  ===========  ====  =====  =  ===========================
tiny            4   8     256          512   1024   2  N(0,1) logits, full softmax
tiny_unit       4   8     256          512   1024   2  as tiny, activations N(0,1)
mixtral         4   8     4096         4096  14336  2  N(0,1) logits, renormalised
qwen3           8   128   2048         4096  1536   8  N(0,1) logits, renormalised
dsv3_skew       8   256   1638x4,410x4 7168  2048   8  Zipf(1.2) Gumbel-top-k
decode_tb32/64  16  128   64           2048  768    8  N(0,1) logits, renormalised
==============  ==  ====  ===========  ====  =====  =  ===========================

Random streams: NumPy PCG64 seeded by ``SeedSequence([seed, 0])`` for routing,
``[seed, 1]`` for activations, ``[seed, 2, g]`` for the weights of global expert
``g`` (gate [f, d], then up [f, d], then down [d, f]), ``[seed, 3, o]`` for the
rows other ranks would return to owner ``o``.  Weights are N(0, 0.02) (0.02 is
the standard deviation).  Conversion to bf16 is torch's round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

__all__ = [
    "MoEConfig", "CONFIGS", "get_config", "owner_token_counts", "routing",
    "activations", "expert_weights", "local_weights", "dispatch",
    "foreign_rows", "to_bf16_bits", "bits_to_float", "random_routing_case",
]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    W: int                 # expert-parallel ranks = token owners
    E: int                 # experts in total, E = W * E_l
    tokens: tuple          # tokens per owner, length W
    d: int                 # hidden size
    f: int                 # expert FFN (intermediate) size
    k: int                 # top-k
    tb_m: int              # row-band height
    route: str = "normal"  # "normal" | "zipf"
    weights: str = "renorm"  # "renorm" | "full_softmax"
    x_std: float = 1.0
    w_std: float = 0.02
    zipf_s: float = 1.2
    seed: int = 0
    rank: int = 0
    mgb: int = 1

    @property
    def E_l(self) -> int:
        return self.E // self.W

    @property
    def N(self) -> int:
        return int(sum(self.tokens))

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


def owner_token_counts(W: int, per_owner: int, skew: Optional[float] = None) -> tuple:
    """Tokens per owner.  With ``skew`` s, owners 0..W/2-1 get weight s and the
    rest weight 1; the total W*per_owner is split by largest remainder."""
    if skew is None:
        return tuple([per_owner] * W)
    w = np.array([skew] * (W // 2) + [1.0] * (W - W // 2))
    total = W * per_owner
    exact = total * w / w.sum()
    base = np.floor(exact).astype(np.int64)
    rem = total - int(base.sum())
    order = np.argsort(-(exact - base), kind="stable")
    base[order[:rem]] += 1
    return tuple(int(x) for x in base)


CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig("tiny", 4, 8, owner_token_counts(4, 256), 512, 1024, 2, 64,
                      weights="full_softmax", x_std=0.02),
    "tiny_unit": MoEConfig("tiny_unit", 4, 8, owner_token_counts(4, 256), 512, 1024, 2, 64,
                           weights="full_softmax", x_std=1.0),
    "mixtral": MoEConfig("mixtral", 4, 8, owner_token_counts(4, 4096), 4096, 14336, 2, 128),
    "qwen3": MoEConfig("qwen3", 8, 128, owner_token_counts(8, 2048), 4096, 1536, 8, 128),
    "dsv3_skew": MoEConfig("dsv3_skew", 8, 256, owner_token_counts(8, 1024, skew=4.0),
                           7168, 2048, 8, 256, route="zipf"),
    "decode_tb32": MoEConfig("decode_tb32", 16, 128, owner_token_counts(16, 64), 2048, 768, 8, 32),
    "decode_tb64": MoEConfig("decode_tb64", 16, 128, owner_token_counts(16, 64), 2048, 768, 8, 64),
}


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float array -> bf16 bit patterns (uint16), round-to-nearest-even (torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_float(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def routing(cfg: MoEConfig):
    """Top-k expert ids [N, k] int32 (global ids, owner-major token order) and
    gate weights [N, k] float32.  Ties in the logits go to the lower expert id."""
    rng = _rng(cfg.seed, 0)
    N, E, k = cfg.N, cfg.E, cfg.k
    if cfg.route == "normal":
        logits = rng.standard_normal((N, E))
    elif cfg.route == "zipf":
        logp = -cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        logp -= np.log(np.exp(logp).sum())
        u = rng.random((N, E))
        u = np.clip(u, 1e-300, 1.0 - 1e-16)
        logits = logp[None, :] - np.log(-np.log(u))
    else:
        raise ValueError(cfg.route)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, ids, axis=1)
    if cfg.weights == "full_softmax":
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        p /= p.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ids, axis=1)
    else:
        m = sel.max(axis=1, keepdims=True)
        p = np.exp(sel - m)
        w = p / p.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


def activations(cfg: MoEConfig) -> np.ndarray:
    """Owner-side token activations [N, d] as bf16 bits (owner-major order)."""
    rng = _rng(cfg.seed, 1)
    x = rng.standard_normal((cfg.N, cfg.d), dtype=np.float32)
    x *= np.float32(cfg.x_std)
    return to_bf16_bits(x)


def expert_weights(cfg: MoEConfig, g: int):
    """(w_gate_up [2f, d], w_down [d, f]) bf16 bits of global expert g.
    Rows 0..f-1 of w_gate_up are the gate projection, rows f..2f-1 the up one."""
    rng = _rng(cfg.seed, 2, g)
    s = np.float32(cfg.w_std)
    gate = rng.standard_normal((cfg.f, cfg.d), dtype=np.float32) * s
    up = rng.standard_normal((cfg.f, cfg.d), dtype=np.float32) * s
    down = rng.standard_normal((cfg.d, cfg.f), dtype=np.float32) * s
    return to_bf16_bits(np.concatenate([gate, up], axis=0)), to_bf16_bits(down)


def local_weights(cfg: MoEConfig, rank: Optional[int] = None):
    """Stacked weights of the experts hosted by ``rank`` (contiguous block
    [rank*E_l, (rank+1)*E_l)): w_gate_up [E_l, 2f, d], w_down [E_l, d, f]."""
    r = cfg.rank if rank is None else rank
    E_l = cfg.E_l
    wgu = np.empty((E_l, 2 * cfg.f, cfg.d), dtype=np.uint16)
    wd = np.empty((E_l, cfg.d, cfg.f), dtype=np.uint16)
    for e in range(E_l):
        a, b = expert_weights(cfg, r * E_l + e)
        wgu[e] = a
        wd[e] = b
    return wgu, wd


def dispatch(cfg: MoEConfig, topk_ids: np.ndarray, x_owner: np.ndarray,
             rank: Optional[int] = None):
    """Token dispatch (the first all-to-all) as seen by ``rank``: every
    (owner, token, slot) triple routed to one of the rank's experts, in
    lexicographic (owner, token, slot) order, carries a copy of the token's
    activation row.  Returns (x_recv [R, d] bf16 bits, token index [R])."""
    r = cfg.rank if rank is None else rank
    lo, hi = r * cfg.E_l, (r + 1) * cfg.E_l
    flat = topk_ids.reshape(-1)
    sel = np.nonzero((flat >= lo) & (flat < hi))[0]
    tok = sel // cfg.k
    return np.ascontiguousarray(x_owner[tok]), tok.astype(np.int64)


def foreign_rows(cfg: MoEConfig, owner: int) -> np.ndarray:
    """Stand-in content for owner ``owner``'s receive buffer [T_o*k, d] (bf16
    bits): the rows the other ranks' experts would return.  The simulated rank
    overwrites its own rows; the rest stay as drawn here."""
    rng = _rng(cfg.seed, 3, owner)
    v = rng.standard_normal((cfg.tokens[owner] * cfg.k, cfg.d), dtype=np.float32)
    return to_bf16_bits(v)


def random_routing_case(rng: np.random.Generator, W: int, E_l: int, k: int,
                        tokens: List[int], hot: Optional[int] = None) -> np.ndarray:
    """Small random routing tables for property tests: k distinct experts per
    token out of W*E_l, optionally biased towards expert ``hot``."""
    E = W * E_l
    N = int(sum(tokens))
    ids = np.empty((N, k), dtype=np.int32)
    for n in range(N):
        if hot is not None and rng.random() < 0.5:
            rest = [g for g in range(E) if g != hot]
            pick = [hot] + list(rng.choice(rest, size=k - 1, replace=False))
        else:
            pick = list(rng.choice(E, size=k, replace=False))
        ids[n] = pick
    return ids
