"""Python binding of libmoe.so: one expert-parallel rank's share of an MoE
layer on one MI355X (owner-aligned layout, remote-first schedule, grouped
SwiGLU FFN with flagged epilogue, consumer copy, gate-weighted scale).

Argument marshalling only: every step runs in the HIP kernels of libmoe.so.
Tensors are torch CUDA tensors (bf16 tensors may be torch.bfloat16 or
int16/uint16 views); streams are torch.cuda.Stream objects (default: the
current stream).  The functions carry the names of the C entry points in
``include/moe.h``.  Importing this package fails loudly when libmoe.so has not
been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ECAPACITY, MOE_EHIP, MOE_ETIMEOUT, MOE_EROUTING, MOE_EUNSUPPORTED = range(7)
MODE_OVERLAP, MODE_SERIAL, MODE_COPY_ONLY, MODE_COPY_ROWS = 0, 1, 2, 3
SIGNAL_TILE, SIGNAL_GROUP = 0, 1

HDR_FIELDS = ["error", "M", "bands", "remote_bands", "segments", "remote_segments",
              "gateup_tiles", "down_tiles", "copy_units", "received_rows", "gateup_row_tiles",
              "down_row_tiles"]


class moe_shape(ctypes.Structure):
    _fields_ = [("world", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("experts_per_rank", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("tb_m", ctypes.c_int32), ("mgb", ctypes.c_int32),
                ("tokens", ctypes.POINTER(ctypes.c_int32)), ("recv_rows", ctypes.c_int64)]


class moe_sizes(ctypes.Structure):
    _fields_ = [("plan_bytes", ctypes.c_size_t), ("rows_cap", ctypes.c_int64),
                ("bands_cap", ctypes.c_int64), ("flags_count", ctypes.c_int64),
                ("recv_rows_self", ctypes.c_int64)]


_VIEW_FIELDS = ["hdr", "c", "grp_off", "m_e", "row_off", "rb", "order", "base",
                "band_expert", "band_dst", "band_src_row", "band_dst_off", "band_valid",
                "seg_first", "seg_nbands", "seg_dst", "seg_dst_off", "seg_src_row", "seg_rows",
                "seg_unit", "src_index", "pos",
                "gu_tile_row", "gu_tile_expert", "dn_tile_row", "dn_tile_expert", "grp_band",
                "sk_counters", "sk_counters_count",
                "crow_off", "grp_crow", "band_crow", "cmp_row", "cmp_src"]


class moe_plan_view(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _VIEW_FIELDS]


class moe_combine_opts(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("consumer_cus", ctypes.c_int32),
                ("consumer_blocks", ctypes.c_int32), ("link_mbps", ctypes.c_int32),
                ("spin_timeout_ns", ctypes.c_int64), ("events", ctypes.c_void_p * 6),
                ("x_recv", ctypes.c_void_p), ("signal", ctypes.c_int32), ("pad", ctypes.c_int32)]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python moe_expert_tile_amd/build.py` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, V = ctypes.POINTER, ctypes.c_int, ctypes.c_void_p
    sig = {
        "moe_status_string": (ctypes.c_char_p, [I]),
        "moe_query_sizes": (I, [P(moe_shape), P(moe_sizes)]),
        "moe_plan_offsets": (I, [P(moe_shape), P(moe_plan_view)]),
        "moe_plan": (I, [P(moe_shape), V, V, V, V, V]),
        "moe_expert_combine": (I, [P(moe_shape), V, V, V, V, V, V, V, ctypes.c_uint32,
                                   P(ctypes.c_void_p), P(moe_combine_opts), V]),
        "moe_expert_combine_noalloc": (I, [P(moe_shape), V, V, V, V, V, V, V, ctypes.c_uint32,
                                           P(ctypes.c_void_p), P(moe_combine_opts), V]),
        "moe_scale": (I, [P(moe_shape), V, V, V, V, V]),
        "moe_device_status": (I, [V, V]),
        "moe_device_cus": (I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ["moe_status_string", "moe_query_sizes", "moe_plan_offsets", "moe_plan",
            "moe_expert_combine", "moe_expert_combine_noalloc", "moe_scale", "moe_device_status",
            "moe_device_cus"]


def library_path() -> str:
    return _LIB_PATH


def status_string(status: int) -> str:
    return _lib.moe_status_string(int(status)).decode()


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoEError(rc, where)


class Shape:
    """moe_shape plus the host token array it points to."""

    def __init__(self, world: int, rank: int, experts_per_rank: int, top_k: int, hidden: int,
                 ffn: int, tb_m: int, tokens: Sequence[int], recv_rows: int, mgb: int = 1):
        self.tokens = list(int(t) for t in tokens)
        self._tok = (ctypes.c_int32 * max(1, len(self.tokens)))(*self.tokens)
        self.c = moe_shape(world, rank, experts_per_rank, top_k, hidden, ffn, tb_m, mgb,
                           ctypes.cast(self._tok, ctypes.POINTER(ctypes.c_int32)), recv_rows)

    def __getattr__(self, name):
        return getattr(self.__dict__["c"], name)

    @property
    def ptr(self):
        return ctypes.byref(self.c)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def moe_query_sizes(shape: Shape) -> Dict[str, int]:
    out = moe_sizes()
    _check(_lib.moe_query_sizes(shape.ptr, ctypes.byref(out)), "moe_query_sizes")
    return {f: int(getattr(out, f)) for f, _ in moe_sizes._fields_}


def moe_plan_offsets(shape: Shape) -> Dict[str, int]:
    out = moe_plan_view()
    _check(_lib.moe_plan_offsets(shape.ptr, ctypes.byref(out)), "moe_plan_offsets")
    return {f: int(getattr(out, f)) for f in _VIEW_FIELDS}


def moe_plan(shape: Shape, topk_ids, x_recv, plan_ws, x_layout, stream=None) -> None:
    _check(_lib.moe_plan(shape.ptr, _ptr(topk_ids), _ptr(x_recv), _ptr(plan_ws), _ptr(x_layout),
                         _stream(stream)), "moe_plan")


def moe_expert_combine(shape: Shape, plan_ws, x_layout, w_gate_up, w_down, h, y, flags, epoch: int,
                       recv: List, mode: int = MODE_OVERLAP, consumer_cus: int = 0,
                       consumer_blocks: int = 0, spin_timeout_ns: int = 0,
                       events: Optional[Sequence] = None, stream=None, x_recv=None,
                       noalloc: bool = False, link_mbps: int = 0, signal: int = SIGNAL_TILE) -> None:
    """x_layout=None with x_recv given: the gate/up GEMM gathers its rows from
    x_recv through the plan's src_index (the layout is never materialized).
    noalloc=True calls moe_expert_combine_noalloc (kernel scratch in the
    library's static device array instead of the plan workspace)."""
    fn = _lib.moe_expert_combine_noalloc if noalloc else _lib.moe_expert_combine
    name = "moe_expert_combine_noalloc" if noalloc else "moe_expert_combine"
    arr = (ctypes.c_void_p * max(1, len(recv)))(*[_ptr(r) for r in recv])
    opts = moe_combine_opts()
    opts.mode = mode
    opts.consumer_cus = consumer_cus
    opts.consumer_blocks = consumer_blocks
    opts.spin_timeout_ns = spin_timeout_ns
    opts.x_recv = _ptr(x_recv)
    opts.link_mbps = int(link_mbps)
    opts.signal = int(signal)
    if events is not None:
        for i, ev in enumerate(events):
            opts.events[i] = None if ev is None else int(ev.cuda_event)
    _check(fn(shape.ptr, _ptr(plan_ws), _ptr(x_layout), _ptr(w_gate_up), _ptr(w_down), _ptr(h), _ptr(y),
              _ptr(flags), int(epoch), ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)),
              ctypes.byref(opts), _stream(stream)), name)


def moe_scale(shape: Shape, plan_ws, recv_self, topk_w, out, stream=None) -> None:
    _check(_lib.moe_scale(shape.ptr, _ptr(plan_ws), _ptr(recv_self), _ptr(topk_w), _ptr(out),
                          _stream(stream)), "moe_scale")


def moe_device_status(plan_ws, stream=None) -> int:
    return int(_lib.moe_device_status(_ptr(plan_ws), _stream(stream)))


def moe_device_cus() -> int:
    return int(_lib.moe_device_cus())


def timing_events(n: int = 6) -> List[torch.cuda.Event]:
    """torch events with timing, already created (recorded once) so that their
    raw handles can be recorded by the library."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    return evs


class RankShare:
    """Device buffers of one rank's share (sized with moe_query_sizes) and the
    three calls of the path.  Buffers are torch allocations; the library
    allocates nothing."""

    def __init__(self, shape: Shape, device="cuda"):
        self.shape = shape
        self.sizes = moe_query_sizes(shape)
        self.offsets = moe_plan_offsets(shape)
        s = shape.c
        dev = torch.device(device)
        rows = self.sizes["rows_cap"]
        self.plan_ws = torch.zeros(self.sizes["plan_bytes"] // 4, dtype=torch.int32, device=dev)
        self.x_layout = torch.empty((rows, s.hidden), dtype=torch.bfloat16, device=dev)
        self.h = torch.empty((rows, s.ffn), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((rows, s.hidden), dtype=torch.bfloat16, device=dev)
        self.flags = torch.zeros(max(1, self.sizes["flags_count"]), dtype=torch.int32, device=dev)
        self.epoch = 0
        self.recv = [torch.zeros((max(1, t * s.top_k), s.hidden), dtype=torch.bfloat16, device=dev)
                     for t in shape.tokens]
        self.out = torch.empty((max(1, shape.tokens[s.rank]), s.hidden), dtype=torch.bfloat16, device=dev)

    def plan(self, topk_ids, x_recv, stream=None, materialize=True):
        """materialize=False: plan metadata only (no layout X); combine must
        then be given x_recv to gather from."""
        moe_plan(self.shape, topk_ids, x_recv, self.plan_ws, self.x_layout if materialize else None, stream)

    def combine(self, w_gate_up, w_down, mode=MODE_OVERLAP, consumer_cus=0, consumer_blocks=0,
                spin_timeout_ns=0, events=None, stream=None, epoch=None, x_recv=None, link_mbps=0,
                signal=SIGNAL_TILE, noalloc=False):
        """x_recv given: gathered rows (the gate/up GEMM reads x_recv through
        src_index instead of the layout X)."""
        if epoch is None:
            epoch = self._next_epoch()
        elif mode in (MODE_OVERLAP, MODE_SERIAL):
            # a compute mode needs a fresh epoch: with one the flags already
            # hold, the consumer could copy rows before they are written
            if not 0 < epoch <= 0xFFFFFFFF or epoch <= self.epoch:
                raise ValueError(f"epoch {epoch} is not above the last one ({self.epoch})")
            self.epoch = epoch
        moe_expert_combine(self.shape, self.plan_ws, self.x_layout if x_recv is None else None, w_gate_up,
                           w_down, self.h, self.y, self.flags, epoch, self.recv, mode, consumer_cus,
                           consumer_blocks, spin_timeout_ns, events, stream, x_recv=x_recv,
                           noalloc=noalloc, link_mbps=link_mbps, signal=signal)

    def _next_epoch(self) -> int:
        """The next epoch; after 2^32 - 1 the flags and the K-split counters
        are zeroed (on the current stream) and the epochs start again at 1."""
        if self.epoch >= 0xFFFFFFFF:
            self.flags.zero_()
            o = self.offsets["sk_counters"] // 4
            self.plan_ws[o:o + 2 * self.offsets["sk_counters_count"]].zero_()
            self.epoch = 0
        self.epoch += 1
        return self.epoch

    def scale(self, topk_w_self, stream=None):
        moe_scale(self.shape, self.plan_ws, self.recv[self.shape.c.rank], topk_w_self, self.out, stream)

    def status(self, stream=None) -> int:
        return moe_device_status(self.plan_ws, stream)

    def header(self) -> Dict[str, int]:
        h = self.plan_ws[self.offsets["hdr"] // 4: self.offsets["hdr"] // 4 + 16].cpu().tolist()
        return {k: h[i] for i, k in enumerate(HDR_FIELDS)}

    def end_stamps(self):
        """(last producer end, last consumer end) of the down-GEMM launch, in
        ticks of the GPU's 100 MHz wall clock (header words 12-15)."""
        o = self.offsets["hdr"] // 4
        w = self.plan_ws[o + 12: o + 16].cpu().numpy().astype(np.uint32).astype(np.uint64)
        return int(w[0] | (w[1] << np.uint64(32))), int(w[2] | (w[3] << np.uint64(32)))

    def array(self, name: str, count: int):
        o = self.offsets[name] // 4
        return self.plan_ws[o:o + count].cpu().numpy()
