"""GPU planner parity: the layout, schedule, combine plan, segments and
owner-side slot table built on the device must equal the oracle's bit for bit
on every workload (and with two segment merge factors), and so must the bytes
of the layout X (tile-signal notes §4.2, §4.4, §4.5, §5.2)."""
import numpy as np
import pytest
import torch

from gpu_helpers import (case, dev_bf16, expected_compacted, expected_plan, host_bits, layout_x, plan_arrays, say,
                         shape_of)

pytestmark = pytest.mark.gpu

WORKLOADS = ["tiny", "mixtral", "qwen3", "dsv3_skew", "decode_tb32", "decode_tb64"]


def run_plan(name, mgb):
    import moe_expert_tile_amd as m
    c = case(name, mgb)
    cfg, pl = c["cfg"], c["plan"]
    say(f"[plan] {name} mgb={mgb} R={pl.R} M={pl.M} bands={pl.n_bands}")
    share = m.RankShare(shape_of(cfg, pl.R))
    ids = torch.from_numpy(c["ids"]).cuda()
    xr = dev_bf16(c["x_recv"])
    share.plan(ids, xr)
    assert share.status() == m.MOE_OK
    return c, share


@pytest.mark.parametrize("mgb", [1, 2])
@pytest.mark.parametrize("name", WORKLOADS)
def test_plan_metadata_bit_exact(name, mgb):
    c, share = run_plan(name, mgb)
    pl = c["plan"]
    hdr = share.header()
    assert hdr["error"] == 0
    assert hdr["M"] == pl.M
    assert hdr["bands"] == pl.n_bands
    assert hdr["remote_bands"] == pl.n_remote
    assert hdr["segments"] == pl.segs["first_band"].shape[0]
    assert hdr["remote_segments"] == pl.n_remote_segs
    assert hdr["received_rows"] == pl.R
    got = plan_arrays(share, hdr)
    exp = expected_plan(pl)
    for k, v in exp.items():
        assert np.array_equal(np.asarray(got[k]).astype(np.int64), np.asarray(v).astype(np.int64)), k
    # the compacted-row tables the GEMMs run on (the layout without padding)
    cx = expected_compacted(pl)
    sizes = {"crow_off": pl.E_l + 1, "grp_crow": pl.E_l * pl.W, "band_crow": pl.n_bands,
             "cmp_row": pl.R, "cmp_src": pl.R}
    for k, v in cx.items():
        g = share.array(k, sizes[k]).astype(np.int64)
        assert np.array_equal(g, np.asarray(v, dtype=np.int64).reshape(-1)), k


@pytest.mark.parametrize("name", WORKLOADS)
def test_layout_bytes_bit_exact(name):
    c, share = run_plan(name, 1)
    pl = c["plan"]
    X = host_bits(share.x_layout[:pl.M])
    assert np.array_equal(X, layout_x(pl, c["x_recv"]))


def test_replanning_reuses_the_workspace():
    """A second plan of a different workload shape in fresh buffers, then the
    first again: results do not depend on what the workspace held."""
    c1, s1 = run_plan("decode_tb32", 1)
    s1.plan_ws.fill_(-7)
    import moe_expert_tile_amd as m
    ids = torch.from_numpy(c1["ids"]).cuda()
    s1.plan(ids, dev_bf16(c1["x_recv"]))
    assert s1.status() == m.MOE_OK
    hdr = s1.header()
    got = plan_arrays(s1, hdr)
    exp = expected_plan(c1["plan"])
    for k, v in exp.items():
        assert np.array_equal(np.asarray(got[k]).astype(np.int64), np.asarray(v).astype(np.int64)), k


def expected_tiles(pl):
    """GEMM row tiles implied by the oracle plan, as (first compacted row,
    expert): gate/up tiles cut the real rows of every X_e (its compacted rows,
    remote groups first and the local group last) into 256-row pieces,
    experts in rule (ii) order; the down tiles are the same pieces in
    schedule order -- first every piece that holds remote rows (experts in
    rule (ii) order), then the pieces of local rows alone (experts
    ascending)."""
    gu_row, gu_exp = [], []
    crow_off = expected_compacted(pl)["crow_off"]
    n_real = [int(crow_off[e + 1] - crow_off[e]) for e in range(pl.E_l)]
    n_remote = [n_real[e] - int(pl.c[e, pl.r]) for e in range(pl.E_l)]
    for e in pl.expert_order:
        for i in range(-(-n_real[e] // 256)):
            gu_row.append(int(crow_off[e]) + 256 * i)
            gu_exp.append(int(e))
    dn = []
    for e in pl.expert_order:
        for i in range(-(-n_remote[e] // 256)):
            dn.append((int(crow_off[e]) + 256 * i, int(e)))
    for e in range(pl.E_l):
        for i in range(-(-n_remote[e] // 256), -(-n_real[e] // 256)):
            dn.append((int(crow_off[e]) + 256 * i, int(e)))
    return gu_row, gu_exp, dn


def expected_group_bands(pl):
    """First band in S of every non-empty (expert, owner) group."""
    out = {}
    for s in range(pl.n_bands):
        key = (int(pl.bands["expert"][s]), int(pl.bands["dst"][s]))
        out.setdefault(key, s)
    return out


def check_tiles(share, pl, hdr):
    gu_row, gu_exp, dn = expected_tiles(pl)
    assert hdr["gateup_row_tiles"] == len(gu_row)
    assert hdr["down_row_tiles"] == len(dn)
    assert share.array("gu_tile_row", len(gu_row)).tolist() == gu_row
    assert share.array("gu_tile_expert", len(gu_row)).tolist() == gu_exp
    got = list(zip(*(share.array(k, len(dn)).tolist() for k in ["dn_tile_row", "dn_tile_expert"])))
    assert got == dn
    o = share.offsets["hdr"] // 4
    crow_off = expected_compacted(pl)["crow_off"]
    n_remote_tiles = sum(1 for row, e in dn if row - crow_off[e] < crow_off[e + 1] - crow_off[e] - pl.c[e, pl.r])
    assert int(share.plan_ws[o + 16]) == n_remote_tiles
    gb = share.array("grp_band", pl.E_l * pl.W).reshape(pl.E_l, pl.W)
    for (e, d), s in expected_group_bands(pl).items():
        assert int(gb[e, d]) == s, (e, d)


@pytest.mark.parametrize("name", WORKLOADS)
def test_gemm_tile_tables(name):
    """The planner's GEMM row-tile tables and group first bands equal the
    ones the oracle plan implies."""
    c, share = run_plan(name, 1)
    check_tiles(share, c["plan"], share.header())


def test_plan_with_band_tables_in_the_workspace():
    """A plan with 4070 bands (bands_cap 4247): the builder's four per-band
    tables (4 x 4248 words, 68 KB) exceed the 64 KB of LDS it may use, so it
    keeps them in the workspace instead.  Metadata, compacted-row tables and
    GEMM tile tables bit-exact as on the other workloads."""
    import moe_expert_tile_amd as m
    import synth
    from oracle import plan as OP
    W, E_l, k, tb, mgb = 16, 8, 8, 32, 2
    tokens = [16000] * W
    cfg = synth.MoEConfig("many_bands", W, W * E_l, tuple(tokens), 256, 256, k, tb, seed=5, mgb=mgb, rank=0)
    ids = synth.random_routing_case(np.random.default_rng(5), W, E_l, k, tokens)
    pl = OP.build_plan(ids, tokens, 0, E_l, tb, mgb)
    rows_cap = pl.R + E_l * (W - 1) * (tb - 1)
    assert rows_cap // tb + E_l * W == 4247 and pl.n_bands == 4070
    say(f"[plan] many_bands R={pl.R} M={pl.M} bands={pl.n_bands}")
    share = m.RankShare(shape_of(cfg, pl.R))
    xr = torch.zeros((pl.R, cfg.d), dtype=torch.bfloat16, device="cuda")
    share.plan(torch.from_numpy(ids).cuda(), xr, materialize=False)
    assert share.status() == m.MOE_OK
    hdr = share.header()
    assert hdr["M"] == pl.M and hdr["bands"] == pl.n_bands and hdr["remote_bands"] == pl.n_remote
    assert hdr["segments"] == pl.segs["first_band"].shape[0] and hdr["remote_segments"] == pl.n_remote_segs
    got = plan_arrays(share, hdr)
    for key, v in expected_plan(pl).items():
        assert np.array_equal(np.asarray(got[key]).astype(np.int64), np.asarray(v).astype(np.int64)), key
    cx = expected_compacted(pl)
    sizes = {"crow_off": E_l + 1, "grp_crow": E_l * W, "band_crow": pl.n_bands, "cmp_row": pl.R, "cmp_src": pl.R}
    for key, v in cx.items():
        assert np.array_equal(share.array(key, sizes[key]).astype(np.int64), np.asarray(v, dtype=np.int64).reshape(-1)), key
    check_tiles(share, pl, hdr)


@pytest.mark.parametrize("W,E_l,k,tokens_per_owner,tb", [
    (4, 256, 8, 1500, 64),    # E_l * W = 1024, the largest group table
    (64, 16, 4, 200, 32),     # the largest world: 64 owners, one wavefront of them
])
def test_plan_at_the_shape_limits(W, E_l, k, tokens_per_owner, tb):
    """Plan metadata, compacted tables and tile tables bit-exact at the
    limits the boundary accepts (W <= 64, W * E_l <= 1024)."""
    import moe_expert_tile_amd as m
    import synth
    from oracle import plan as OP
    tokens = [tokens_per_owner + 7 * o for o in range(W)]
    rank = W - 1
    cfg = synth.MoEConfig("limits", W, W * E_l, tuple(tokens), 256, 256, k, tb, seed=11, mgb=2, rank=rank)
    ids = synth.random_routing_case(np.random.default_rng(11), W, E_l, k, tokens)
    pl = OP.build_plan(ids, tokens, rank, E_l, tb, 2)
    say(f"[plan] limits W={W} E_l={E_l} R={pl.R} M={pl.M} bands={pl.n_bands}")
    share = m.RankShare(shape_of(cfg, pl.R))
    xr = torch.zeros((max(pl.R, 1), cfg.d), dtype=torch.bfloat16, device="cuda")
    share.plan(torch.from_numpy(ids).cuda(), xr, materialize=False)
    assert share.status() == m.MOE_OK
    hdr = share.header()
    assert hdr["M"] == pl.M and hdr["bands"] == pl.n_bands and hdr["remote_bands"] == pl.n_remote
    assert hdr["segments"] == pl.segs["first_band"].shape[0] and hdr["remote_segments"] == pl.n_remote_segs
    got = plan_arrays(share, hdr)
    for key, v in expected_plan(pl).items():
        assert np.array_equal(np.asarray(got[key]).astype(np.int64), np.asarray(v).astype(np.int64)), key
    cx = expected_compacted(pl)
    sizes = {"crow_off": E_l + 1, "grp_crow": E_l * W, "band_crow": pl.n_bands, "cmp_row": pl.R, "cmp_src": pl.R}
    for key, v in cx.items():
        assert np.array_equal(share.array(key, sizes[key]).astype(np.int64), np.asarray(v, dtype=np.int64).reshape(-1)), key
    check_tiles(share, pl, hdr)
