"""GPU planner parity: the layout, schedule, combine plan, segments and
owner-side slot table built on the device must equal the oracle's bit for bit
on every workload (and with two segment merge factors), and so must the bytes
of the layout X (tile-signal notes §4.2, §4.4, §4.5, §5.2)."""
import numpy as np
import pytest
import torch

from gpu_helpers import case, dev_bf16, expected_plan, host_bits, layout_x, plan_arrays, say, shape_of

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
