"""GPU parity of the expert FFN, the combine and the scale on every workload.

* FFN (tile-signal notes §5.1; SwiGLU expert): h and y of every layout row
  (small workloads) or of sampled rows — every band's first and last valid
  row, padding rows, X_e boundaries, random rows — against the oracle in
  float64, within |gpu - ref| <= 2e-2 + 1e-2 |ref|; every padding row of y
  is exactly zero (§4.2 step 2).
* Combine (§4.5, §5.2): with the receive buffers pre-filled with other ranks'
  rows, exactly the plan's rows change and each is a bit-exact copy of its
  layout row; repeated overlapped epochs without a flag reset, with y
  poisoned by NaN before each call, copy exactly their own y and give the
  same y again; serial and overlapped y agree within the tolerance.
* Per-row copy (the §4.3 alternative to the layout, as an ablation): the
  remote rows copied one per wavefront give the segment copy's bits.
* Gathered rows: the gate/up GEMM reading the layout's rows from x_recv
  through src_index instead of a materialized X gives the same bits.
* Scale (§2.2 step 5): sampled tokens of the rank's own output against the
  oracle, whose receive rows come from the oracle's own FFN.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import (ATOL, RTOL, case, dev_bf16, h_rows, host_bits, layout_x, oracle_ffn_rows,
                         oracle_sample, owner_slice, rows_of, sample_rows, say, shape_of, tol_ratio, weights)
from oracle import combine as OC
from oracle import scale as OS
from oracle import bf16 as OB

pytestmark = pytest.mark.gpu

WORKLOADS = ["tiny", "tiny_unit", "mixtral", "qwen3", "dsv3_skew", "decode_tb32", "decode_tb64"]
_runs = {}


def planned(name, mode):
    """Plan + expert_combine of the workload in the given mode (cached)."""
    import moe_expert_tile_amd as m
    key = (name, mode)
    if key in _runs:
        return _runs[key]
    c = case(name)
    cfg, pl = c["cfg"], c["plan"]
    say(f"[path] {name} mode={mode} M={pl.M}")
    share = m.RankShare(shape_of(cfg, pl.R))
    share.plan(torch.from_numpy(c["ids"]).cuda(), dev_bf16(c["x_recv"]))
    wgu, wd = weights(name)
    wgu_d, wd_d = dev_bf16(wgu), dev_bf16(wd)
    for o in range(cfg.W):
        share.recv[o].copy_(dev_bf16(synth.foreign_rows(cfg, o)))
    share.combine(wgu_d, wd_d, mode=mode)
    assert share.status() == m.MOE_OK
    _runs.clear()
    _runs[key] = (c, share, wgu_d, wd_d)
    return _runs[key]


@pytest.mark.parametrize("name", WORKLOADS)
def test_ffn_rows_match_oracle(name):
    import moe_expert_tile_amd as m
    c, share, _, _ = planned(name, m.MODE_SERIAL)
    pl = c["plan"]
    rows, h_ref, y_ref = oracle_sample(name)
    h, h_ref = h_rows(share, pl, rows, h_ref)
    y = rows_of(share.y, rows)
    scale_aware = name == "tiny"
    rh = tol_ratio(h, h_ref, scale_aware)
    ry = tol_ratio(y, y_ref, scale_aware)
    say(f"[ffn] {name} rows={rows.size} worst h {rh:.3f} y {ry:.3f} (1.0 = tolerance)")
    assert rh <= 1.0 and ry <= 1.0
    if name != "tiny":
        # the unscaled bar too
        assert tol_ratio(y, y_ref) <= 1.0
    pad = np.nonzero(pl.src_index < 0)[0]
    if pad.size:
        yp = share.y.index_select(0, torch.from_numpy(pad).cuda())
        assert bool((yp == 0).all())


@pytest.mark.parametrize("name", WORKLOADS)
def test_combine_writes_exactly_the_plan(name):
    import moe_expert_tile_amd as m
    c, share, _, _ = planned(name, m.MODE_OVERLAP)
    cfg, pl = c["cfg"], c["plan"]
    Y = host_bits(share.y[:pl.M])
    written = OC.written_rows(pl)
    for o in range(cfg.W):
        exp = synth.foreign_rows(cfg, o)
        dst, src = written[o]
        exp[dst] = Y[src]
        got = host_bits(share.recv[o][: exp.shape[0]])
        assert np.array_equal(got, exp), f"owner {o}"


@pytest.mark.parametrize("name", ["tiny_unit", "qwen3", "dsv3_skew", "decode_tb32", "decode_tb64"])
@pytest.mark.parametrize("serial", [True, False])
def test_every_band_head_and_tail_flag_is_set(name, serial):
    """After a compute call both flags of every band -- head and tail, for
    every column tile -- equal the call's epoch, remote and local bands alike
    (a down tile may end inside a band, so a band's two flags may come from
    two tiles; the consumer only waits on remote bands, so this is what shows
    that no local band's flag is missed), and no flag word past the plan's
    bands is written."""
    import moe_expert_tile_amd as m
    c, share, _, _ = planned(name, m.MODE_SERIAL if serial else m.MODE_OVERLAP)
    hdr = share.header()
    n_used = hdr["down_tiles"]
    assert n_used == 2 * hdr["bands"] * (share.shape.hidden // 256)
    f = share.flags.cpu().numpy().view(np.uint32)
    assert np.all(f[:n_used] == share.epoch), np.nonzero(f[:n_used] != share.epoch)[0][:8]
    assert np.all(f[n_used:] == 0)


@pytest.mark.parametrize("name", ["tiny_unit", "mixtral", "qwen3", "decode_tb32", "dsv3_skew"])
def test_per_row_copy_equals_the_segment_copy(name):
    """The per-row ablation of the copy (the notes' alternative to the
    owner-aligned layout, §4.3: every row routed on its own at transfer
    time): with the remote owners' buffers refilled, copying the remote rows
    one per wavefront leaves every buffer bit for bit as the plan applied to
    y -- the same result as the segment consumer."""
    import moe_expert_tile_amd as m
    c, share, _, _ = planned(name, m.MODE_OVERLAP)
    cfg, pl = c["cfg"], c["plan"]
    for o in range(cfg.W):
        if o != cfg.rank:
            share.recv[o].copy_(dev_bf16(synth.foreign_rows(cfg, o)))
    share.combine(None, None, mode=m.MODE_COPY_ROWS, epoch=share.epoch)
    assert share.status() == m.MOE_OK
    Y = host_bits(share.y[:pl.M])
    written = OC.written_rows(pl)
    for o in range(cfg.W):
        exp = synth.foreign_rows(cfg, o)
        dst, src = written[o]
        exp[dst] = Y[src]
        assert np.array_equal(host_bits(share.recv[o][: exp.shape[0]]), exp), f"owner {o}"


@pytest.mark.parametrize("name,blocks", [("mixtral", 16), ("qwen3", 8), ("qwen3", 256), ("dsv3_skew", 16),
                                         ("decode_tb32", 4)])
def test_copy_with_few_consumer_workgroups(name, blocks):
    """The standalone consumer on a small grid (each workgroup copies many
    units, two in flight): after a serial call, with the receive buffers
    refilled, a copy-only call with `blocks` workgroups writes exactly the
    plan applied to y."""
    import moe_expert_tile_amd as m
    c, share, _, _ = planned(name, m.MODE_SERIAL)
    cfg, pl = c["cfg"], c["plan"]
    for o in range(cfg.W):
        share.recv[o].copy_(dev_bf16(synth.foreign_rows(cfg, o)))
    share.combine(None, None, mode=m.MODE_COPY_ONLY, epoch=share.epoch, consumer_blocks=blocks)
    assert share.status() == m.MOE_OK
    Y = host_bits(share.y[:pl.M])
    written = OC.written_rows(pl)
    for o in range(cfg.W):
        exp = synth.foreign_rows(cfg, o)
        if o != cfg.rank:   # the rank's own rows come from the down GEMM, not the copy
            dst, src = written[o]
            exp[dst] = Y[src]
        assert np.array_equal(host_bits(share.recv[o][: exp.shape[0]]), exp), f"owner {o}"


@pytest.mark.parametrize("name", ["tiny_unit", "mixtral", "qwen3", "decode_tb32", "dsv3_skew"])
def test_overlapped_combine_over_epochs(name):
    """Overlapped calls, each with y poisoned by NaN and the receive buffers
    refilled first: every call's buffers equal the plan applied to that call's
    own y (a consumer that read a tile before its flag would copy NaN or stale
    rows), y is identical across epochs (the stream-K fixup sums in a fixed
    order), and y matches the serial mode's within the tolerance -- bit for bit
    where neither mode splits tiles along K (the overlapped down GEMM has 16
    fewer producers, so the two modes may split different tail tiles)."""
    import moe_expert_tile_amd as m
    c, share, wgu_d, wd_d = planned(name, m.MODE_SERIAL)
    cfg, pl = c["cfg"], c["plan"]
    y_serial = host_bits(share.y[:pl.M])
    written = OC.written_rows(pl)
    y_first = None
    for it in range(3):
        share.y.fill_(float("nan"))
        for o in range(cfg.W):
            share.recv[o].copy_(dev_bf16(synth.foreign_rows(cfg, o)))
        share.combine(wgu_d, wd_d, mode=m.MODE_OVERLAP)
        assert share.status() == m.MOE_OK
        Y = host_bits(share.y[:pl.M])
        for o in range(cfg.W):
            exp = synth.foreign_rows(cfg, o)
            dst, src = written[o]
            exp[dst] = Y[src]
            assert np.array_equal(host_bits(share.recv[o][: exp.shape[0]]), exp), (it, o)
        if y_first is None:
            y_first = Y
        else:
            assert np.array_equal(Y, y_first), it
    # the overlapped y straight against the oracle, and against the serial y
    rows, _, y_ref = oracle_sample(name)
    ratio = tol_ratio(y_first[rows], y_ref)
    say(f"[overlap] {name} rows={rows.size} worst y {ratio:.3f} against the oracle")
    assert ratio <= 1.0
    assert tol_ratio(y_first, y_serial, name == "tiny") <= 1.0
    if name in ("tiny_unit", "decode_tb32"):
        assert np.array_equal(y_first, y_serial)


@pytest.mark.parametrize("name,mgb,cus", [("qwen3", 1, 8), ("qwen3", 4, 64), ("decode_tb32", 4, 8),
                                          ("decode_tb64", 2, 64), ("tiny_unit", 4, 128)])
def test_overlapped_combine_consumer_budgets(name, mgb, cus):
    """The overlapped combine with other consumer budgets and segment merge
    factors (§5.2, §5.3): copy units are claimed in schedule order by the
    consumer workgroups and by producers out of tiles; over two epochs, with
    y poisoned by NaN before each, the receive buffers are exactly the plan
    (built with this mgb) applied to that call's own y."""
    import moe_expert_tile_amd as m
    c = case(name, mgb)
    cfg, pl = c["cfg"], c["plan"]
    say(f"[budget] {name} mgb={mgb} consumer_cus={cus}")
    share = m.RankShare(shape_of(cfg.replace(mgb=mgb), pl.R))
    share.plan(torch.from_numpy(c["ids"]).cuda(), dev_bf16(c["x_recv"]))
    wgu, wd = weights(name)
    wgu_d, wd_d = dev_bf16(wgu), dev_bf16(wd)
    hdr = share.header()
    assert hdr["segments"] == pl.segs["first_band"].shape[0]
    written = OC.written_rows(pl)
    for it in range(2):
        share.y.fill_(float("nan"))
        for o in range(cfg.W):
            share.recv[o].copy_(dev_bf16(synth.foreign_rows(cfg, o)))
        share.combine(wgu_d, wd_d, mode=m.MODE_OVERLAP, consumer_cus=cus)
        assert share.status() == m.MOE_OK
        Y = host_bits(share.y[:pl.M])
        for o in range(cfg.W):
            exp = synth.foreign_rows(cfg, o)
            dst, src = written[o]
            exp[dst] = Y[src]
            assert np.array_equal(host_bits(share.recv[o][: exp.shape[0]]), exp), (it, o)


@pytest.mark.parametrize("name", ["tiny_unit", "mixtral", "qwen3", "dsv3_skew", "decode_tb32", "decode_tb64"])
def test_gathered_rows_equal_the_layout_path(name):
    """Gathered A rows: a plan that does not materialize the layout X, and a
    gate/up GEMM that reads every layout row from x_recv through src_index
    (padding rows as zeros), give h, y and receive buffers bit-identical to
    the materialized layout's in the serial mode, and in the overlapped mode
    receive buffers that are exactly the plan applied to their own y; the
    layout buffer is never written."""
    import moe_expert_tile_amd as m
    c, share, wgu_d, wd_d = planned(name, m.MODE_SERIAL)
    cfg, pl = c["cfg"], c["plan"]
    H, Y = host_bits(share.h[:pl.R]), host_bits(share.y[:pl.M])
    recv_ref = [host_bits(r) for r in share.recv]
    written = OC.written_rows(pl)
    g = m.RankShare(shape_of(cfg, pl.R))
    g.x_layout.fill_(float("nan"))
    xr = dev_bf16(c["x_recv"])
    g.plan(torch.from_numpy(c["ids"]).cuda(), xr, materialize=False)
    rows, h_ref, y_ref = oracle_sample(name)
    for mode in (m.MODE_SERIAL, m.MODE_OVERLAP):
        for o in range(cfg.W):
            g.recv[o].copy_(dev_bf16(synth.foreign_rows(cfg, o)))
        g.h.fill_(float("nan"))
        g.y.fill_(float("nan"))
        g.combine(wgu_d, wd_d, mode=mode, x_recv=xr)
        assert g.status() == m.MOE_OK
        # gathered h and y straight against the oracle ...
        rh = tol_ratio(*h_rows(g, pl, rows, h_ref))
        ry = tol_ratio(rows_of(g.y, rows), y_ref)
        say(f"[gathered] {name} mode={mode} worst h {rh:.3f} y {ry:.3f} against the oracle")
        assert rh <= 1.0 and ry <= 1.0
        # ... and bit for bit against the materialized layout's
        assert np.array_equal(host_bits(g.h[:pl.R]), H), mode
        y = host_bits(g.y[:pl.M])
        if mode == m.MODE_SERIAL:
            assert np.array_equal(y, Y)
            for o in range(cfg.W):
                assert np.array_equal(host_bits(g.recv[o]), recv_ref[o]), o
        else:
            assert tol_ratio(y, Y) <= 1.0
            for o in range(cfg.W):
                exp = synth.foreign_rows(cfg, o)
                dst, src = written[o]
                exp[dst] = y[src]
                assert np.array_equal(host_bits(g.recv[o][: exp.shape[0]]), exp), o
    assert bool(torch.isnan(g.x_layout[: min(pl.M, 512)].float()).all())
    del g


@pytest.mark.parametrize("name", WORKLOADS)
def test_scale_matches_oracle(name):
    import moe_expert_tile_amd as m
    c, share, _, _ = planned(name, m.MODE_OVERLAP)
    cfg, pl = c["cfg"], c["plan"]
    r = cfg.rank
    w_r = c["w"][owner_slice(cfg, r)]
    share.scale(torch.from_numpy(w_r).cuda())
    assert share.status() == m.MOE_OK
    T = cfg.tokens[r]
    rng = np.random.default_rng(1)
    toks = np.arange(T) if T <= 1024 else np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 256)]))
    # receive rows these tokens read: the rank's own band rows come from the
    # oracle FFN of their layout rows, the rest are the other ranks' rows
    dst, src = OC.written_rows(pl)[r]
    from_layout = dict(zip(dst.tolist(), src.tolist()))
    need = np.unique(pl.pos[toks].reshape(-1))
    recv_r = synth.foreign_rows(cfg, r)
    lay_rows = np.array([from_layout[q] for q in need if q in from_layout], dtype=np.int64)
    if lay_rows.size:
        X = layout_x(pl, c["x_recv"])
        _, y_ref = oracle_ffn_rows(name, pl, X, lay_rows)
        for q, yy in zip([q for q in need if q in from_layout], y_ref):
            recv_r[q] = yy
    out_ref = OS.scale(recv_r, w_r, pl.pos, toks)
    out = host_bits(share.out.index_select(0, torch.from_numpy(toks).cuda()))
    ratio = tol_ratio(out, out_ref, scale_aware=(name == "tiny"))
    say(f"[scale] {name} tokens={toks.size} worst {ratio:.3f}")
    assert ratio <= 1.0


@pytest.mark.parametrize("name", ["tiny_unit", "qwen3", "dsv3_skew"])
def test_scale_alone_within_rounding_bound(name):
    """Scale on fixed receive rows (no GEMM in between).  The GPU sums k fp32
    products in order; the oracle sums in float64 and rounds once.  Their
    difference is bounded by one bf16 ulp of the result plus the fp32
    accumulation error, k * 2^-23 * sum_j |w_j x_j| (standard bound for
    recursive summation with fused multiply-add)."""
    import moe_expert_tile_amd as m
    c, share, _, _ = planned(name, m.MODE_OVERLAP)
    cfg, pl = c["cfg"], c["plan"]
    r = cfg.rank
    recv_r = synth.foreign_rows(cfg, r)
    share.recv[r].copy_(dev_bf16(recv_r))
    w_r = c["w"][owner_slice(cfg, r)]
    share.scale(torch.from_numpy(w_r).cuda())
    assert share.status() == m.MOE_OK
    out = OB.from_bits(host_bits(share.out[: cfg.tokens[r]]))
    ref_bits = OS.scale(recv_r, w_r, pl.pos)
    ref = OB.from_bits(ref_bits)
    absum = np.einsum("tk,tkd->td", np.abs(w_r.astype(np.float64)), np.abs(OB.from_bits(recv_r[pl.pos])))
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.maximum(np.abs(ref), np.abs(out)), 1e-38))[1] - 8)
    bound = ulp + cfg.k * 2.0 ** -23 * absum
    excess = float((np.abs(out - ref) / bound).max())
    say(f"[scale-bound] {name} worst {excess:.3f}, max ulps {int(OB.ulp_distance(host_bits(share.out[: cfg.tokens[r]]), ref_bits).max())}")
    assert excess <= 1.0


@pytest.mark.parametrize("name,signal,link", [("tiny_unit", 1, 2000), ("qwen3", 1, 153000), ("mixtral", 1, 0),
                                              ("decode_tb32", 0, 153000), ("dsv3_skew", 1, 153000),
                                              ("decode_tb64", 1, 20000)])
def test_paced_and_group_signalled_combine(name, signal, link):
    """The consumer behind an emulated link per destination (link_mbps) and
    with group-batched ready counters instead of per-band flags (signal 1;
    the Perseus page's decoupled signalling, one signal per destination
    group), in the overlapped and the serial mode, over two epochs with y
    poisoned by NaN first: y is bit for bit the per-band, unpaced y of the
    same mode, and the receive buffers are exactly the plan applied to it."""
    import moe_expert_tile_amd as m
    c = case(name)
    cfg, pl = c["cfg"], c["plan"]
    wgu, wd = weights(name)
    wgu_d, wd_d = dev_bf16(wgu), dev_bf16(wd)
    written = OC.written_rows(pl)
    say(f"[signal] {name} signal={signal} link_mbps={link}")
    for mode in (m.MODE_OVERLAP, m.MODE_SERIAL):
        ref = m.RankShare(shape_of(cfg, pl.R))
        ref.plan(torch.from_numpy(c["ids"]).cuda(), dev_bf16(c["x_recv"]))
        ref.combine(wgu_d, wd_d, mode=mode)
        assert ref.status() == m.MOE_OK
        y_ref = host_bits(ref.y[:pl.M])
        sh = m.RankShare(shape_of(cfg, pl.R))
        sh.plan(torch.from_numpy(c["ids"]).cuda(), dev_bf16(c["x_recv"]))
        for it in range(2):
            sh.y.fill_(float("nan"))
            for o in range(cfg.W):
                sh.recv[o].copy_(dev_bf16(synth.foreign_rows(cfg, o)))
            sh.combine(wgu_d, wd_d, mode=mode, signal=signal, link_mbps=link)
            assert sh.status() == m.MOE_OK
            Y = host_bits(sh.y[:pl.M])
            assert np.array_equal(Y, y_ref), (mode, it)
            for o in range(cfg.W):
                exp = synth.foreign_rows(cfg, o)
                dst, src = written[o]
                exp[dst] = Y[src]
                assert np.array_equal(host_bits(sh.recv[o][: exp.shape[0]]), exp), (mode, it, o)
        del ref, sh


def test_paced_copy_takes_at_least_the_link_time():
    """With flags already set, the copy alone at 2000 MB/s per destination
    lasts at least (bytes to the busiest destination) / rate: the emulated
    links bound it, not the memory."""
    import moe_expert_tile_amd as m
    c, share, _, _ = planned("tiny_unit", m.MODE_SERIAL)
    cfg, pl = c["cfg"], c["plan"]
    sg = pl.segs
    per_dst = np.zeros(cfg.W)
    for q in range(pl.n_remote_segs):
        per_dst[int(sg["dst"][q])] += int(sg["rows"][q]) * cfg.d * 2
    rate = 2000e6
    floor_s = per_dst.max() / rate
    times = []
    for _ in range(3):
        e0, e1 = m.timing_events(2)
        e0.record()
        share.combine(None, None, mode=m.MODE_COPY_ONLY, epoch=share.epoch, link_mbps=2000)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    assert share.status() == m.MOE_OK
    say(f"[paced] busiest destination {per_dst.max() / 1e3:.0f} KB: floor {floor_s * 1e6:.1f} us, "
        f"copy {min(times) * 1e6:.1f} us")
    assert min(times) >= 0.9 * floor_s
    assert min(times) <= 10 * floor_s + 1e-3
