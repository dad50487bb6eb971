"""The C ABI without a GPU: the library loads, exports every entry point that
include/moe.h declares, sizes follow the padding bound of the tile-signal
notes (§4.3: at most (W-1)(tb_M-1) padding rows per local expert), and the
host-side validation rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "moe_expert_tile_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    import moe_expert_tile_amd as m
    assert sorted(m.EXPORTED) == names


def _shape(**kw):
    import moe_expert_tile_amd as m
    base = dict(world=4, rank=0, experts_per_rank=2, top_k=2, hidden=512, ffn=1024, tb_m=64,
                tokens=[256] * 4, recv_rows=500, mgb=1)
    base.update(kw)
    return m.Shape(**base)


def test_sizes_follow_the_padding_bound():
    import moe_expert_tile_amd as m
    for W, E_l, tb, R in [(4, 2, 64, 500), (8, 32, 256, 46000), (16, 8, 32, 511), (1, 3, 128, 77)]:
        s = _shape(world=W, rank=W - 1, experts_per_rank=E_l, tb_m=tb, tokens=[64] * W,
                   recv_rows=min(R, 64 * W * 2), top_k=2)
        z = m.moe_query_sizes(s)
        R = s.recv_rows
        assert z["rows_cap"] == R + E_l * (W - 1) * (tb - 1)
        assert z["bands_cap"] == z["rows_cap"] // tb + E_l * W
        assert z["recv_rows_self"] == 64 * 2
        assert z["plan_bytes"] % 256 == 0
        off = m.moe_plan_offsets(s)
        vals = sorted(v for k, v in off.items() if not k.endswith("_count"))
        assert all(v % 256 == 0 for v in vals)
        assert len(set(vals)) == len(vals)
        assert max(vals) < z["plan_bytes"]


@pytest.mark.parametrize("bad", [
    dict(world=0), dict(world=65), dict(rank=4), dict(rank=-1), dict(experts_per_rank=0),
    dict(experts_per_rank=300), dict(top_k=0), dict(top_k=9), dict(hidden=500), dict(hidden=128),
    dict(ffn=1000), dict(tb_m=48), dict(tb_m=16), dict(tb_m=512), dict(mgb=0),
    dict(tokens=[256, -1, 256, 256]), dict(recv_rows=-1), dict(recv_rows=4 * 256 * 2 + 1),
])
def test_bad_shapes_are_rejected(bad):
    import moe_expert_tile_amd as m
    with pytest.raises(m.MoEError) as ei:
        m.moe_query_sizes(_shape(**bad))
    assert ei.value.status == m.MOE_EINVAL


def test_bad_pointers_are_rejected_before_any_hip_call():
    import moe_expert_tile_amd as m
    s = _shape()
    good = 1 << 20  # never dereferenced: validation fails first
    with pytest.raises(m.MoEError) as ei:
        m.moe_plan(s, good, good, 0, good, stream=0)
    assert ei.value.status == m.MOE_EINVAL
    with pytest.raises(m.MoEError) as ei:
        m.moe_plan(s, good, good + 8, good, good, stream=0)        # misaligned x_recv
    assert ei.value.status == m.MOE_EINVAL
    with pytest.raises(m.MoEError) as ei:
        m.moe_expert_combine(s, good, good, good, good, good, good, good, 0, [good] * 4, stream=0)
    assert ei.value.status == m.MOE_EINVAL                        # epoch 0
    with pytest.raises(m.MoEError) as ei:
        m.moe_expert_combine(s, good, good, good, good, good, good, good, 1, [good] * 4,
                             consumer_cus=12, stream=0)
    assert ei.value.status == m.MOE_EINVAL                        # not a multiple of 8
    with pytest.raises(m.MoEError) as ei:
        m.moe_expert_combine(s, good, good, good, good, good, good, good, 1, [good] * 4,
                             consumer_cus=16, consumer_blocks=17, stream=0)
    assert ei.value.status == m.MOE_EINVAL                        # more consumer workgroups than CUs
    for bad_mode in (-1, 4):
        with pytest.raises(m.MoEError) as ei:
            m.moe_expert_combine(s, good, good, good, good, good, good, good, 1, [good] * 4,
                                 mode=bad_mode, stream=0)
        assert ei.value.status == m.MOE_EINVAL                    # no such mode
    with pytest.raises(m.MoEError) as ei:
        m.moe_expert_combine(s, good, None, None, None, None, None, good, 1, [good] * 4,
                             mode=m.MODE_COPY_ROWS, stream=0)
    assert ei.value.status == m.MOE_EINVAL                        # per-row copy without y
    with pytest.raises(m.MoEError) as ei:
        m.moe_expert_combine(s, good, good, good, good, good, good, good, 1, [good, 0, good, good],
                             stream=0)
    assert ei.value.status == m.MOE_EINVAL                        # null receive buffer
    with pytest.raises(m.MoEError) as ei:
        m.moe_expert_combine(s, good, None, good, good, good, good, good, 1, [good] * 4, stream=0)
    assert ei.value.status == m.MOE_EINVAL                        # no layout and nothing to gather from
    with pytest.raises(m.MoEError) as ei:
        m.moe_expert_combine(s, good, None, good, good, good, good, good, 1, [good] * 4, stream=0,
                             x_recv=good + 4)
    assert ei.value.status == m.MOE_EINVAL                        # misaligned x_recv to gather from
    big = _shape(hidden=65536, ffn=128, tokens=[8192] * 4, recv_rows=16384, top_k=2)
    with pytest.raises(m.MoEError) as ei:
        m.moe_expert_combine(big, good, None, good, good, good, good, good, 1, [good] * 4, stream=0,
                             x_recv=good)
    assert ei.value.status == m.MOE_EINVAL                        # R*d*2 = 2^31 bytes: too large to gather
    for kw in (dict(link_mbps=999), dict(link_mbps=-1), dict(signal=2), dict(signal=-1),
               dict(signal=m.SIGNAL_GROUP, mode=m.MODE_COPY_ROWS)):
        for noalloc in (False, True):
            with pytest.raises(m.MoEError) as ei:
                m.moe_expert_combine(s, good, good, good, good, good, good, good, 1, [good] * 4, stream=0,
                                     noalloc=noalloc, **kw)
            assert ei.value.status == m.MOE_EINVAL, kw               # link too slow, no such signal,
                                                                     # per-row copy without tile flags
    with pytest.raises(m.MoEError) as ei:
        m.moe_scale(s, good, good, good, good + 2, stream=0)
    assert ei.value.status == m.MOE_EINVAL
    assert m.moe_device_status(0, stream=0) == m.MOE_EINVAL


def test_status_strings():
    import moe_expert_tile_amd as m
    for code in range(7):
        assert m.status_string(code)
    assert m.status_string(99) == "unknown status"


def test_stream_k_scratch_only_where_a_gemm_can_split():
    """The plan workspace holds stream-K partial sums only when one of the
    GEMMs is long enough in K to be split (32 K steps of 64 at least): none
    for d = 512, f = 1024 (8 and 16 steps), 512 slots of 256 KB for d = 4096."""
    import moe_expert_tile_amd as m
    small = m.moe_query_sizes(_shape())
    assert small["plan_bytes"] < (1 << 20)
    big = m.moe_query_sizes(_shape(hidden=4096, ffn=14336))
    assert big["plan_bytes"] >= 512 * 256 * 256 * 4
    off = m.moe_plan_offsets(_shape())
    assert off["sk_counters_count"] == 512 and off["sk_counters"] % 256 == 0


def test_epochs_of_the_binding():
    """RankShare.combine refuses, before any library call, an explicit epoch
    that is not above the last one in a compute mode (its flags would already
    read as ready), and the automatic epoch skips 0 on wrap-around after
    zeroing the flags and the K-split counters."""
    import torch
    import moe_expert_tile_amd as m
    sh = m.RankShare(_shape(), device="cpu")
    sh.epoch = 7
    for e in (7, 3, 0, 1 << 32):
        with pytest.raises(ValueError):
            sh.combine(None, None, mode=m.MODE_OVERLAP, epoch=e)
        with pytest.raises(ValueError):
            sh.combine(None, None, mode=m.MODE_SERIAL, epoch=e)
    assert sh.epoch == 7
    sh.epoch = 0xFFFFFFFF
    sh.flags.fill_(5)
    o = sh.offsets["sk_counters"] // 4
    sh.plan_ws[o:o + 1024].fill_(9)
    assert sh._next_epoch() == 1
    assert int(sh.flags.abs().sum()) == 0 and int(sh.plan_ws[o:o + 1024].abs().sum()) == 0
    assert sh._next_epoch() == 2
