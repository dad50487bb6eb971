"""Whole-layer emulation and edge cases on the GPU.

* Every rank's share of a small layer runs on the one GPU into shared owner
  receive buffers (the W ranks are W buffers in HBM); every owner then scales
  its tokens, and the result is compared with the MoE output computed token by
  token from its definition by the oracle (gate-weighted sum of the top-k
  experts' FFN outputs; tile-signal notes §2.1, §2.2).  This exercises the
  receive offsets of all ranks' plans against each other.
* Edge cases: no tokens at all, ragged owners (one empty), a single rank
  (no remote bands), a hot expert, k = E, a band height that is not a power of
  two, band heights that do not divide the 256-row GEMM tile, the largest
  band height, a large merge factor, and 16 or 64 owners (up to 64 owner
  groups in one down tile).
* Failure handling forced from the host, with every kernel exiting normally:
  an expert id out of range and a received-row count that disagrees with the
  routing are reported as MOE_EROUTING and later kernels do nothing; a
  consumer waiting for an epoch no producer set gives MOE_ETIMEOUT within
  its bound.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import dev_bf16, host_bits, say, tol_ratio
from oracle import brute
from oracle import combine as OC
from oracle import ffn as OF
from oracle import plan as OP
from oracle import scale as OS

pytestmark = pytest.mark.gpu


def _shape(cfg, rank, R):
    import moe_expert_tile_amd as m
    return m.Shape(cfg.W, rank, cfg.E_l, cfg.k, cfg.d, cfg.f, cfg.tb_m, cfg.tokens, R, mgb=cfg.mgb)


def run_layer(cfg, ids, w, x_owner, mode):
    """All W ranks' shares into shared receive buffers, then every owner's
    scale.  Returns the output [N, d] bf16 bits."""
    import moe_expert_tile_amd as m
    shares = []
    recv = [torch.zeros((max(1, t * cfg.k), cfg.d), dtype=torch.bfloat16, device="cuda") for t in cfg.tokens]
    ids_d = torch.from_numpy(ids).cuda()
    for r in range(cfg.W):
        x_recv, _ = synth.dispatch(cfg, ids, x_owner, rank=r)
        sh = m.RankShare(_shape(cfg, r, x_recv.shape[0]))
        sh.recv = recv
        sh.plan(ids_d, dev_bf16(x_recv) if x_recv.shape[0] else torch.zeros((1, cfg.d), dtype=torch.bfloat16,
                                                                            device="cuda"))
        wgu, wd = synth.local_weights(cfg, r)
        sh.combine(dev_bf16(wgu), dev_bf16(wd), mode=mode)
        assert sh.status() == m.MOE_OK
        shares.append(sh)
    off = OP.owner_offsets(cfg.tokens)
    out = np.zeros((cfg.N, cfg.d), np.uint16)
    for o in range(cfg.W):
        if cfg.tokens[o] == 0:
            continue
        shares[o].scale(torch.from_numpy(np.ascontiguousarray(w[off[o]:off[o + 1]])).cuda())
        assert shares[o].status() == m.MOE_OK
        out[off[o]:off[o + 1]] = host_bits(shares[o].out[: cfg.tokens[o]])
    return out


@pytest.mark.parametrize("name,mode", [("tiny", 0), ("tiny_unit", 0), ("tiny_unit", 1)])
def test_full_layer_equals_definition(name, mode):
    cfg = synth.get_config(name)
    ids, w = synth.routing(cfg)
    x = synth.activations(cfg)
    say(f"[layer] {name} mode={mode}")
    out = run_layer(cfg, ids, w, x, mode)
    cache = {}
    def weight_of(g):
        if g not in cache:
            cache[g] = synth.expert_weights(cfg, g)
        return cache[g]
    ref = brute.moe_output(x, ids, w, weight_of)
    ratio = tol_ratio(out, ref, scale_aware=(name == "tiny"))
    say(f"[layer] {name} worst {ratio:.3f}")
    assert ratio <= 1.0


def _custom(W, E_l, k, tokens, d=256, f=256, tb=32, mgb=1, seed=0, hot=None, rank=0, fixed=None):
    """A small layer; `fixed` (k expert ids) routes every token to the same
    experts instead of drawing them."""
    assert tb % 32 == 0 and 32 <= tb <= 256 and d % 256 == 0 and f % 128 == 0
    cfg = synth.MoEConfig("custom", W, W * E_l, tuple(tokens), d, f, k, tb, seed=seed, mgb=mgb, rank=rank)
    rng = np.random.default_rng(seed)
    if fixed is not None:
        assert len(fixed) == k and len(set(fixed)) == k
        ids = np.tile(np.asarray(fixed, dtype=np.int32), (int(sum(tokens)), 1))
    else:
        ids = synth.random_routing_case(rng, W, E_l, k, list(tokens), hot=hot)
    w = rng.random((cfg.N, k)).astype(np.float32)
    return cfg, ids, w


EDGE_CASES = {
    "empty": dict(W=4, E_l=2, k=2, tokens=[0, 0, 0, 0]),
    "ragged": dict(W=4, E_l=3, k=3, tokens=[5, 0, 300, 17], mgb=3, rank=2),
    "single_rank": dict(W=1, E_l=4, k=2, tokens=[200]),
    "hot_expert": dict(W=3, E_l=2, k=2, tokens=[150, 90, 40], hot=0),
    "k_equals_E": dict(W=2, E_l=2, k=4, tokens=[33, 70], rank=1),
    "tb96": dict(W=3, E_l=2, k=2, tokens=[120, 80, 100], tb=96, mgb=2),
    "tb256_wide": dict(W=5, E_l=1, k=1, tokens=[300, 10, 260, 0, 513], tb=256, d=512, f=384),
    # band heights that do not divide 256: the down GEMM's 256-row tiles end
    # inside bands, whose head and tail flags then come from two tiles
    # (tb192 with K = 1024, long enough to split the single round along K)
    "tb160": dict(W=3, E_l=2, k=2, tokens=[460, 190, 530], tb=160, mgb=2, rank=1),
    "tb192": dict(W=3, E_l=2, k=2, tokens=[600, 400, 500], tb=192, f=1024, mgb=2),
    "tb224": dict(W=4, E_l=1, k=2, tokens=[500, 350, 0, 610], tb=224, mgb=3, rank=3),
    # many owner groups in one down tile: the epilogue takes one wavefront
    # lane per group (64 at most), each with its own padding and flags
    "w64_tb32": dict(W=64, E_l=1, k=4, tokens=[60] * 64, tb=32, mgb=2, rank=5),
    "w16_tb64": dict(W=16, E_l=4, k=4, tokens=[100 + 13 * o for o in range(16)], tb=64, rank=15),
    # every group an exact multiple of tb_M: no padding row anywhere (M = R)
    "exact_multiples": dict(W=3, E_l=2, k=2, tokens=[64, 128, 96], fixed=[1, 0]),
    # the rank routes nothing to itself: its local group is empty
    "local_empty": dict(W=3, E_l=2, k=2, tokens=[200, 0, 150], rank=1),
    # every row from one remote owner
    "one_owner": dict(W=4, E_l=2, k=2, tokens=[0, 0, 333, 0]),
}


@pytest.mark.parametrize("case_name", list(EDGE_CASES))
def test_edge_case_rank_share(case_name):
    """Plan bit-exact; every layout row's y within tolerance; the receive
    buffers hold exactly the plan's rows; the rank's output within tolerance
    of the oracle fed with the same receive buffer; with gathered rows (no
    layout X), and with group-batched signals, the same y and receive
    buffers bit for bit."""
    import moe_expert_tile_amd as m
    p = dict(EDGE_CASES[case_name])
    cfg, ids, w = _custom(**p)
    r = cfg.rank
    x = synth.activations(cfg)
    x_recv, _ = synth.dispatch(cfg, ids, x)
    pl = OP.build_plan(ids, cfg.tokens, r, cfg.E_l, cfg.tb_m, cfg.mgb)
    say(f"[edge] {case_name} R={pl.R} M={pl.M} bands={pl.n_bands}")
    sh = m.RankShare(_shape(cfg, r, pl.R))
    # other ranks' rows (finite, distinct): any stray write would change them
    sentinel = [synth.foreign_rows(cfg, o) if cfg.tokens[o] else np.zeros((1, cfg.d), np.uint16)
                for o in range(cfg.W)]
    for o in range(cfg.W):
        sh.recv[o].copy_(dev_bf16(sentinel[o]))
    ids_d = torch.from_numpy(ids).cuda() if ids.size else torch.zeros(1, dtype=torch.int32, device="cuda")
    xr = dev_bf16(x_recv) if pl.R else torch.zeros((1, cfg.d), dtype=torch.bfloat16, device="cuda")
    sh.plan(ids_d, xr)
    wgu, wd = synth.local_weights(cfg, r)
    sh.combine(dev_bf16(wgu), dev_bf16(wd), mode=m.MODE_OVERLAP, consumer_cus=16)
    assert sh.status() == m.MOE_OK
    hdr = sh.header()
    assert hdr["M"] == pl.M and hdr["bands"] == pl.n_bands and hdr["remote_bands"] == pl.n_remote
    if pl.M:
        assert np.array_equal(sh.array("src_index", pl.M), pl.src_index)
        X = OC.layout_x(pl, x_recv)
        _, y_ref = OF.layout_rows(pl, X, wgu, wd, np.arange(pl.M))
        y = host_bits(sh.y[: pl.M])
        assert tol_ratio(y, y_ref) <= 1.0
    Y = host_bits(sh.y[: max(pl.M, 1)])
    written = OC.written_rows(pl)
    for o in range(cfg.W):
        exp = sentinel[o].copy()
        dst, src = written[o]
        exp[dst] = Y[src]
        assert np.array_equal(host_bits(sh.recv[o]), exp), o
    T = cfg.tokens[r]
    if T:
        w_r = np.ascontiguousarray(w[OP.owner_offsets(cfg.tokens)[r]:][:T])
        sh.scale(torch.from_numpy(w_r).cuda())
        assert sh.status() == m.MOE_OK
        recv_r = host_bits(sh.recv[r])
        ref = OS.scale(recv_r, w_r, pl.pos)
        assert tol_ratio(host_bits(sh.out[:T]), ref) <= 1.0
    # the same share with gathered rows (no layout X): the same y and the same
    # receive buffers, bit for bit
    recv_mat = [host_bits(t) for t in sh.recv]
    for o in range(cfg.W):
        sh.recv[o].copy_(dev_bf16(sentinel[o]))
    sh.y.fill_(float("nan"))
    sh.plan(ids_d, xr, materialize=False)
    sh.combine(dev_bf16(wgu), dev_bf16(wd), mode=m.MODE_OVERLAP, consumer_cus=16,
               x_recv=xr if pl.R else None)
    assert sh.status() == m.MOE_OK
    if pl.M:
        assert np.array_equal(host_bits(sh.y[: pl.M]), Y[: pl.M])
    for o in range(cfg.W):
        assert np.array_equal(host_bits(sh.recv[o]), recv_mat[o]), o
    # and with group-batched signals (one ready counter per (expert,
    # destination) group, raised by the band heads and tails each tile
    # holds): the same y and receive buffers, bit for bit
    for o in range(cfg.W):
        sh.recv[o].copy_(dev_bf16(sentinel[o]))
    sh.y.fill_(float("nan"))
    sh.plan(ids_d, xr)
    sh.combine(dev_bf16(wgu), dev_bf16(wd), mode=m.MODE_OVERLAP, consumer_cus=16, signal=m.SIGNAL_GROUP)
    assert sh.status() == m.MOE_OK
    if pl.M:
        assert np.array_equal(host_bits(sh.y[: pl.M]), Y[: pl.M])
    for o in range(cfg.W):
        assert np.array_equal(host_bits(sh.recv[o]), recv_mat[o]), o


def test_bad_expert_id_is_reported_and_nothing_runs():
    import moe_expert_tile_amd as m
    cfg, ids, w = _custom(W=2, E_l=2, k=2, tokens=[40, 40])
    x = synth.activations(cfg)
    x_recv, _ = synth.dispatch(cfg, ids, x)
    sh = m.RankShare(_shape(cfg, 0, x_recv.shape[0]))
    bad = ids.copy()
    bad[7, 1] = cfg.E          # out of range
    sh.y.fill_(1.0)
    sh.plan(torch.from_numpy(bad).cuda(), dev_bf16(x_recv))
    wgu, wd = synth.local_weights(cfg, 0)
    sh.combine(dev_bf16(wgu), dev_bf16(wd), mode=m.MODE_OVERLAP, consumer_cus=8)
    assert sh.status() == m.MOE_EROUTING
    assert bool((sh.y == 1.0).all())                   # the GEMMs did nothing
    # a good plan in the same workspace clears the error
    sh.plan(torch.from_numpy(ids).cuda(), dev_bf16(x_recv))
    sh.combine(dev_bf16(wgu), dev_bf16(wd), mode=m.MODE_SERIAL)
    assert sh.status() == m.MOE_OK


def test_received_row_count_mismatch_is_reported():
    import moe_expert_tile_amd as m
    cfg, ids, w = _custom(W=2, E_l=2, k=2, tokens=[40, 40])
    x = synth.activations(cfg)
    x_recv, _ = synth.dispatch(cfg, ids, x)
    sh = m.RankShare(_shape(cfg, 0, x_recv.shape[0] - 1))
    sh.plan(torch.from_numpy(ids).cuda(), dev_bf16(x_recv))
    assert sh.status() == m.MOE_EROUTING


def test_consumer_wait_is_bounded():
    """Only the consumer runs, for an epoch no producer ever set: it gives up
    after its 2 ms bound and reports MOE_ETIMEOUT."""
    import moe_expert_tile_amd as m
    cfg, ids, w = _custom(W=3, E_l=2, k=2, tokens=[64, 64, 64])
    x = synth.activations(cfg)
    x_recv, _ = synth.dispatch(cfg, ids, x)
    sh = m.RankShare(_shape(cfg, 0, x_recv.shape[0]))
    sh.plan(torch.from_numpy(ids).cuda(), dev_bf16(x_recv))
    assert sh.status() == m.MOE_OK
    sh.combine(None, None, mode=m.MODE_COPY_ONLY, spin_timeout_ns=2_000_000, epoch=12345)
    assert sh.status() == m.MOE_ETIMEOUT
