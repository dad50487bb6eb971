"""Benchmark: one expert-parallel rank's share of an MoE layer on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
moe_plan (owner-aligned layout, remote-first schedule, combine plan, layout
X) -> moe_expert_combine (gate/up GEMM + SwiGLU, down GEMM with tile flags in
parallel with the consumer copy on reserved CUs) -> moe_scale.  Inputs are
resident in HBM before the timed region.  The default workload is the
largest one, the DeepSeek-V3-like skewed layer (W=8 ranks, 256 experts with
32 local, owner token counts 1638x4 + 410x4, d=7168, f=2048, top-8 with
Zipf(1.2) expert popularity, tb_M=256), rank 0's share: rank 0 hosts the
32 hottest experts, so it is the busiest rank.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode overlap|serial]
                    [--consumer-cus C] [--mgb B] [--no-cpu-baseline]

Prints one JSON line.  value = tokens/s = (N / W) / (time per step), with N
the layer's tokens over all W owners: the per-GPU rate of the layer if every
rank took as long as rank 0.  routed rows/s = R / (time per step).  The
timed steps carry no events; per-stage times (means in stages_us, median and
10th / 90th percentiles in stage_spread_us) come from as many steps again
with events around every call.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s
METRIC = "MoE-layer tokens/s on 1 MI355X; grouped-GEMM TFLOP/s & combine GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3_skew")
    ap.add_argument("--mode", default="overlap", choices=["overlap", "serial"])
    ap.add_argument("--consumer-cus", type=int, default=16)
    ap.add_argument("--mgb", type=int, default=None,
                    help="segment merge factor (bands per middle segment); default: the workload's (1)")
    ap.add_argument("--link-gbps", type=float, default=0.0,
                    help="emulated link per destination rank for the consumer's copies, GB/s (0: memory speed; "
                         "one xGMI link is ~153)")
    ap.add_argument("--signal", default="tile", choices=["tile", "group"],
                    help="per-band tile flags, or one ready counter per (expert, destination) group")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gathered", action="store_true",
                    help="skip the gathered-rows variant (profiling runs that count one kind of gate/up launch)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 1 GiB device to device 3 times (a plain copy of known "
                         "size, to scale the FETCH_SIZE / WRITE_SIZE counters of a profiling run)")
    return ap.parse_args()


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"gateup_gemm_{workload}_traffic.txt")


GEMM_SOURCES = [os.path.join(ROOT, "moe_expert_tile_amd", "csrc", n)
                for n in ("gemm.hip", "consume.h", "moe_internal.h")]


def gemm_code_digest():
    """sha256 of the GEMM kernel's sources with comments and whitespace
    removed: counters taken on one revision stay valid across comment-only
    edits and become void on any change to the code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        src = open(path).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
        h.update(b"\0")
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per gate/up GEMM launch from the committed counter summary,
    or None when there is none for this workload or the kernel source has
    changed since the counters were taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_code_sha256") != gemm_code_digest():
        return None
    f_fetch = float(kv["copy_bytes"]) / (1024.0 * float(kv["copy_fetch_kib"]))
    f_write = float(kv["copy_bytes"]) / (1024.0 * float(kv["copy_write_kib"]))
    return 1024.0 * (float(kv["gateup_fetch_kib"]) * f_fetch + float(kv["gateup_write_kib"]) * f_write)


def dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def algorithmic(cfg, R, M, n_seg_rows, gu_rows, dn_rows):
    """Work per call (the rank-0 share) in the units the rooflines use.  The
    GEMMs' algorithmic flops count the R real rows only: padding rows carry
    no data (the gate/up GEMM never computes them; the down GEMM writes zeros
    for them).  The rows the kernels run through their MFMAs, ragged tile
    tails and padding included, are reported beside as executed flops."""
    d, f, k, T_r = cfg.d, cfg.f, cfg.k, cfg.tokens[cfg.rank]
    N = cfg.N
    return {
        "gateup_flop": 4.0 * d * f * R,
        "down_flop": 2.0 * d * f * R,
        "gateup_flop_executed": 4.0 * d * f * gu_rows,
        "down_flop_executed": 2.0 * d * f * dn_rows,
        "useful_flop": 6.0 * d * f * R,
        "plan_bytes": 4.0 * N * k + 2.0 * d * R + 2.0 * d * M + 4.0 * M + 4.0 * T_r * k,
        "combine_bytes": 4.0 * d * n_seg_rows,   # valid rows read + written
        "scale_bytes": 2.0 * d * k * T_r + 2.0 * d * T_r + 8.0 * k * T_r,
        # the bytes the gate/up GEMM must move at least: X's real rows and
        # every local expert's W_gate_up read once, h written once
        "gateup_bytes": 2.0 * d * R + 4.0 * cfg.E_l * f * d + 2.0 * f * R,
    }


def host_info():
    """Threads the oracle's BLAS may use on this host (the CPU share: the
    affinity mask, capped by OMP_NUM_THREADS when that is set), the BLAS
    library numpy calls, and the CPU model."""
    affinity = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    threads = min(affinity, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else affinity
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = "%s %s (%s)" % (libs[0].get("internal_api"), libs[0].get("version"),
                                   os.path.basename(libs[0].get("filepath", "")))
    except Exception:  # pragma: no cover
        pass
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return {"threads": threads, "affinity_cpus": affinity, "blas": blas, "cpu_model": model}


def cpu_baseline(cfg, ids, w, x_recv, wgu, wd, budget_s):
    """The oracle as it stands on the host, on a bounded sample: the full plan,
    the FFN on a sample of layout rows (extrapolated to all M rows), the
    combine and the scale of the rank's tokens.  Same unit as the GPU line:
    (N / W) tokens per step over the summed stage times."""
    from oracle import combine as OC, ffn as OF, plan as OP, scale as OS
    info = host_info()
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=info["threads"], user_api="blas")
    except Exception:  # pragma: no cover
        limiter = contextlib.nullcontext()
    with limiter:
        t0 = time.perf_counter()
        pl = OP.build_plan(ids, cfg.tokens, cfg.rank, cfg.E_l, cfg.tb_m, cfg.mgb)
        X = OC.layout_x(pl, x_recv)
        t_plan = time.perf_counter() - t0
        rng = np.random.default_rng(0)
        n = 64
        t_ffn_rows, rows_done = 0.0, 0
        while t_ffn_rows < budget_s * 0.6 and rows_done < pl.M:
            n = min(n, pl.M - rows_done)
            rows = rng.integers(0, pl.M, n)
            t1 = time.perf_counter()
            OF.layout_rows(pl, X, wgu, wd, rows)
            t_ffn_rows += time.perf_counter() - t1
            rows_done += n
            n = min(2 * n, 1024)
        t_ffn = t_ffn_rows / max(rows_done, 1) * pl.M
        Y = np.zeros((pl.M, cfg.d), np.uint16)
        recv = [np.zeros((t * cfg.k, cfg.d), np.uint16) for t in cfg.tokens]
        t2 = time.perf_counter()
        recv = OC.apply(pl, Y, recv)
        t_comb = time.perf_counter() - t2
        t3 = time.perf_counter()
        OS.scale(recv[cfg.rank], w[: cfg.tokens[cfg.rank]], pl.pos)
        t_scale = time.perf_counter() - t3
    total = t_plan + t_ffn + t_comb + t_scale
    return {
        "value": round((cfg.N / cfg.W) / total, 3), "unit": "tokens/s", "cores": int(info["threads"]),
        "kind": "oracle",
        "sample": f"full plan+layout ({t_plan:.2f}s), FFN on {rows_done} random of {pl.M} layout rows "
                  f"({t_ffn_rows:.2f}s, extrapolated to {t_ffn:.1f}s), full combine ({t_comb:.2f}s) "
                  f"and scale ({t_scale:.2f}s); float64 NumPy; one step = {total:.1f}s",
        "affinity_cpus": info["affinity_cpus"], "blas": info["blas"], "cpu_model": info["cpu_model"],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs one GPU only (the W ranks are emulated as HBM partitions on it); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_expert_tile_amd as m
    import synth

    cfg = synth.get_config(args.workload) if args.mgb is None else synth.get_config(args.workload, mgb=args.mgb)
    ids, w = synth.routing(cfg)
    x_owner = synth.activations(cfg)
    x_recv, _ = synth.dispatch(cfg, ids, x_owner)
    wgu, wd = synth.local_weights(cfg)
    R = x_recv.shape[0]
    T_r = cfg.tokens[cfg.rank]

    share = m.RankShare(m.Shape(cfg.W, cfg.rank, cfg.E_l, cfg.k, cfg.d, cfg.f, cfg.tb_m, cfg.tokens, R,
                                mgb=cfg.mgb))
    ids_d = torch.from_numpy(ids).cuda()
    xr_d = dev_bf16(x_recv, torch)
    wgu_d, wd_d = dev_bf16(wgu, torch), dev_bf16(wd, torch)
    w_r = torch.from_numpy(np.ascontiguousarray(w[:T_r])).cuda()
    for o in range(cfg.W):
        share.recv[o].copy_(dev_bf16(synth.foreign_rows(cfg, o), torch))
    mode = m.MODE_OVERLAP if args.mode == "overlap" else m.MODE_SERIAL
    link_mbps = int(round(args.link_gbps * 1000))
    signal = m.SIGNAL_GROUP if args.signal == "group" else m.SIGNAL_TILE
    cx = dict(link_mbps=link_mbps, signal=signal)   # how the consumer waits and copies
    stream = torch.cuda.current_stream()

    n_ev = args.steps
    ev_plan = [m.timing_events(2) for _ in range(n_ev)]
    ev_comb = [m.timing_events(6) for _ in range(n_ev)]
    ev_scale = [m.timing_events(2) for _ in range(n_ev)]

    def step(i=None):
        if i is not None:
            ev_plan[i][0].record(stream)
        share.plan(ids_d, xr_d)
        if i is not None:
            ev_plan[i][1].record(stream)
        share.combine(wgu_d, wd_d, mode=mode, consumer_cus=args.consumer_cus,
                      events=ev_comb[i] if i is not None else None, **cx)
        if i is not None:
            ev_scale[i][0].record(stream)
        share.scale(w_r)
        if i is not None:
            ev_scale[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = share.status()
    if st != m.MOE_OK:
        raise SystemExit(f"device status after warmup: {m.status_string(st)}")
    # the timed steps carry no events (an event record between two kernels
    # can cost GPU time); the per-stage times come from the same number of
    # steps again, each ABI call between its own pair of events
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    st = share.status()
    if st != m.MOE_OK:
        raise SystemExit(f"device status after timed steps: {m.status_string(st)}")
    ms = elapsed / args.steps * 1e3

    def avg(pairs):
        return float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e-3

    def spread(pairs):
        # median and 10th / 90th percentiles over the instrumented steps, us
        v = np.array([a.elapsed_time(b) for a, b in pairs]) * 1e3
        return {"median": round(float(np.median(v)), 2), "p10": round(float(np.percentile(v, 10)), 2),
                "p90": round(float(np.percentile(v, 90)), 2)}

    t_plan = avg([(e[0], e[1]) for e in ev_plan])
    t_gu = avg([(e[0], e[1]) for e in ev_comb])
    t_dn = avg([(e[2], e[3]) for e in ev_comb])
    t_cons = avg([(e[4], e[5]) for e in ev_comb])
    t_ec = avg([(e[0], ev_scale[i][0]) for i, e in enumerate(ev_comb)])
    t_scale = avg([(e[0], e[1]) for e in ev_scale])
    stage_spread = {
        "plan": spread([(e[0], e[1]) for e in ev_plan]),
        "gateup_gemm": spread([(e[0], e[1]) for e in ev_comb]),
        "down_gemm": spread([(e[2], e[3]) for e in ev_comb]),
        "expert_combine": spread([(e[0], ev_scale[i][0]) for i, e in enumerate(ev_comb)]),
        "scale": spread([(e[0], e[1]) for e in ev_scale]),
        "step": spread([(ev_plan[i][0], ev_scale[i][1]) for i in range(n_ev)]),
    }
    hdr = share.header()
    M = hdr["M"]
    # the consumer moves the remote segments (local rows are written by the
    # down GEMM's epilogue)
    nrs = hdr["remote_segments"]
    seg_rows = int(share.array("seg_rows", nrs).sum()) if nrs else 0
    # rows the GEMMs' tiles hold: 256-row tiles over every expert's real
    # rows, in both GEMMs; the 32-row blocks of a tile that hold no row are
    # not multiplied, but counted here
    gu_rows = 256 * hdr["gateup_row_tiles"]
    dn_rows = 256 * hdr["down_row_tiles"]
    work = algorithmic(cfg, R, M, seg_rows, gu_rows, dn_rows)

    # Short kernels: 20 back-to-back launches between two events on the
    # stream they run on, so the per-launch event overhead does not count.
    # A full serial combine (~3 ms of GPU work) goes first, so the host has
    # queued all 20 launches before the first one starts: the interval is the
    # GPU's back-to-back time, not the host's launch rate.
    def amortized(fn, n=20):
        share.combine(wgu_d, wd_d, mode=m.MODE_SERIAL, **cx)
        e0, e1 = m.timing_events(2)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    t_plan_k = amortized(lambda: share.plan(ids_d, xr_d))
    t_scale_k = amortized(lambda: share.scale(w_r))
    # standalone consumer: flags already equal the last epoch, all CUs
    t_copy = amortized(lambda: share.combine(None, None, mode=m.MODE_COPY_ONLY, epoch=share.epoch, **cx))
    # the per-row ablation of the copy (every remote row routed and copied
    # on its own, as without the owner-aligned layout), all CUs
    t_rows = amortized(lambda: share.combine(None, None, mode=m.MODE_COPY_ROWS, epoch=share.epoch)) \
        if signal == m.SIGNAL_TILE else None
    # ... and with only the consumer's CU budget of workgroups
    t_copy_budget = amortized(lambda: share.combine(None, None, mode=m.MODE_COPY_ONLY, epoch=share.epoch,
                                                    consumer_blocks=args.consumer_cus, **cx))

    # The same kernels with a cold Infinity Cache: each launch follows a read
    # of a 1 GiB buffer (4x the 256 MB cache; a read leaves no dirty lines to
    # write back during the kernel) and is timed alone by its own pair of
    # events (it is queued while the read runs); median of n launches.
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")

    def amortized_cold(fn, n=15):
        evs = [m.timing_events(2) for _ in range(n)]
        for a, b in evs:
            flush_buf.max()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e-3

    t_plan_cold = amortized_cold(lambda: share.plan(ids_d, xr_d))
    t_scale_cold = amortized_cold(lambda: share.scale(w_r))
    t_copy_cold = amortized_cold(lambda: share.combine(None, None, mode=m.MODE_COPY_ONLY, epoch=share.epoch, **cx))
    t_rows_cold = amortized_cold(lambda: share.combine(None, None, mode=m.MODE_COPY_ROWS, epoch=share.epoch)) \
        if signal == m.SIGNAL_TILE else None
    # context for the copy: the runtime's own device-to-device copy of as
    # many bytes as the consumer reads (and writes), timed the same way
    half = int(work["combine_bytes"]) // 2
    t_dev_copy_cold = None
    if half > 0:
        cp_src = torch.empty(half, dtype=torch.uint8, device="cuda")
        cp_dst = torch.empty_like(cp_src)
        t_dev_copy_cold = amortized_cold(lambda: cp_dst.copy_(cp_src))
        del cp_src, cp_dst
    del flush_buf
    st = share.status()
    if st != m.MOE_OK:
        raise SystemExit(f"device status after standalone launches: {m.status_string(st)}")

    # Overlap (the notes' overlap ratio): the consumer's tail after the last
    # producer workgroup of the down GEMM ends, from the device's own end
    # stamps (100 MHz clock), against the standalone copy time; and the same
    # step in the serial mode (GEMMs, then the copy on all CUs).
    tail = None
    if mode == m.MODE_OVERLAP:
        tails = []
        for _ in range(5):
            share.plan(ids_d, xr_d)
            share.combine(wgu_d, wd_d, mode=mode, consumer_cus=args.consumer_cus, **cx)
            torch.cuda.synchronize()
            end_prod, end_cons = share.end_stamps()
            tails.append(max(0, end_cons - end_prod) * 1e-8)
        tail = float(np.median(tails))
    # the serial mode's warm-up steps carry events: the GEMMs alone, the
    # down GEMM on every CU with no consumer beside it
    n_serial = 10
    ev_ser = [m.timing_events(6) for _ in range(3)]
    for i in range(3):
        share.plan(ids_d, xr_d)
        share.combine(wgu_d, wd_d, mode=m.MODE_SERIAL, events=ev_ser[i], **cx)
        share.scale(w_r)
    torch.cuda.synchronize()
    t_gu_ser = float(np.median([e[0].elapsed_time(e[1]) for e in ev_ser])) * 1e-3
    t_dn_ser = float(np.median([e[2].elapsed_time(e[3]) for e in ev_ser])) * 1e-3
    t0s = time.perf_counter()
    for _ in range(n_serial):
        share.plan(ids_d, xr_d)
        share.combine(wgu_d, wd_d, mode=m.MODE_SERIAL, **cx)
        share.scale(w_r)
    torch.cuda.synchronize()
    ms_serial = (time.perf_counter() - t0s) / n_serial * 1e3

    # The same step with gathered rows: the plan builds the metadata only and
    # the gate/up GEMM reads each layout row from x_recv through src_index,
    # so the layout X is never materialized (no gather kernel, no pad fill).
    def step_gathered():
        share.plan(ids_d, xr_d, materialize=False)
        share.combine(wgu_d, wd_d, mode=mode, consumer_cus=args.consumer_cus, x_recv=xr_d, **cx)
        share.scale(w_r)

    ms_gathered = t_plan_meta = None
    if not args.no_gathered:
        for _ in range(3):
            step_gathered()
        torch.cuda.synchronize()
        n_g = max(5, args.steps // 2)
        t0g = time.perf_counter()
        for _ in range(n_g):
            step_gathered()
        torch.cuda.synchronize()
        ms_gathered = (time.perf_counter() - t0g) / n_g * 1e3
        t_plan_meta = amortized(lambda: share.plan(ids_d, xr_d, materialize=False))
        st = share.status()
        if st != m.MOE_OK:
            raise SystemExit(f"device status after gathered-row steps: {m.status_string(st)}")

    gu_tflops = work["gateup_flop"] / t_gu
    # producer workgroups of the down GEMM, one per CU: the CUs the consumer
    # does not hold in the overlapped launch (rounded down to whole XCDs)
    n_prod = (256 - args.consumer_cus) // 8 * 8 if mode == m.MODE_OVERLAP else 256
    tokens_per_rank = cfg.N / cfg.W   # N / W: the layer's tokens per rank
    result = {
        "metric": METRIC,
        "value": round(tokens_per_rank / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: rank {cfg.rank} share of W={cfg.W} ranks, E={cfg.E} experts "
                        f"({cfg.E_l} local), {cfg.tokens[0]} tokens per owner, d={cfg.d}, f={cfg.f} SwiGLU, "
                        f"top-{cfg.k}, tb_M={cfg.tb_m}, mgb={cfg.mgb}",
            "mode": args.mode, "consumer_cus": args.consumer_cus, "link_gbps": args.link_gbps or None,
            "signal": args.signal, "N": cfg.N, "W": cfg.W, "R": R, "M": M,
            "padding_pct": round(100.0 * (M - R) / max(M, 1), 2),
        },
        "roofline": {
            "kernel": "gate/up grouped GEMM + SwiGLU (grouped_gemm_kernel, gate/up instance)",
            "algorithmic": "4*d*f*R flops per launch (R real rows; no padding row is computed)",
            "bound": "mfma", "achieved": round(gu_tflops / 1e12, 2), "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": round(gu_tflops / PEAK_BF16, 4), "traffic": measured_traffic(args.workload),
            "traffic_algorithmic": work["gateup_bytes"],
        },
        "stages_us": {
            "plan_in_step": round(t_plan * 1e6, 2), "gateup_gemm": round(t_gu * 1e6, 2),
            "down_gemm": round(t_dn * 1e6, 2), "consumer": round(t_cons * 1e6, 2),
            "expert_combine": round(t_ec * 1e6, 2), "scale_in_step": round(t_scale * 1e6, 2),
            "plan_back_to_back": round(t_plan_k * 1e6, 2), "scale_back_to_back": round(t_scale_k * 1e6, 2),
            "consumer_standalone_back_to_back": round(t_copy * 1e6, 2),
            "consumer_standalone_at_budget": round(t_copy_budget * 1e6, 2),
            "consumer_standalone_cold_cache": round(t_copy_cold * 1e6, 2),
            "consumer_per_row_back_to_back": round(t_rows * 1e6, 2) if t_rows else None,
            "consumer_per_row_cold_cache": round(t_rows_cold * 1e6, 2) if t_rows_cold else None,
            "device_copy_same_bytes_cold_cache": round(t_dev_copy_cold * 1e6, 2) if t_dev_copy_cold else None,
            "scale_cold_cache": round(t_scale_cold * 1e6, 2),
            "plan_cold_cache": round(t_plan_cold * 1e6, 2),
            # serial mode (median of 3 steps): each GEMM alone on every CU
            "gateup_gemm_serial": round(t_gu_ser * 1e6, 2),
            "down_gemm_serial": round(t_dn_ser * 1e6, 2),
        },
        # the instrumented steps' stage times (the means above) as median
        # and 10th / 90th percentiles; "step" runs from the plan's first
        # event to the scale's last, so it includes the event records
        "stage_spread_us": stage_spread,
        "rates": {
            # primary bandwidth figures: each launch alone after a 1 GiB read
            # (a cold Infinity Cache), so the bytes come from HBM
            "plan_frac_hbm_cold": round(work["plan_bytes"] / t_plan_cold / PEAK_HBM, 4),
            "combine_frac_hbm_cold": round(work["combine_bytes"] / t_copy_cold / PEAK_HBM, 4),
            "scale_frac_hbm_cold": round(work["scale_bytes"] / t_scale_cold / PEAK_HBM, 4),
            "gateup_TFLOPs": round(gu_tflops / 1e12, 2),
            "down_TFLOPs": round(work["down_flop"] / t_dn / 1e12, 2),
            "down_frac_mfma": round(work["down_flop"] / t_dn / PEAK_BF16, 4),
            # the overlapped down GEMM against the peak of the CUs its
            # producers hold (the launch's other workgroups are the consumer)
            "down_frac_mfma_producer_cus": round(work["down_flop"] / t_dn / (PEAK_BF16 * n_prod / 256), 4),
            "down_frac_mfma_serial": round(work["down_flop"] / t_dn_ser / PEAK_BF16, 4),
            "gateup_frac_mfma_executed": round(work["gateup_flop_executed"] / t_gu / PEAK_BF16, 4),
            "down_frac_mfma_executed": round(work["down_flop_executed"] / t_dn / PEAK_BF16, 4),
            "plan_GBs_cold": round(work["plan_bytes"] / t_plan_cold / 1e9, 1),
            "combine_GBs_cold": round(work["combine_bytes"] / t_copy_cold / 1e9, 1),
            "scale_GBs_cold": round(work["scale_bytes"] / t_scale_cold / 1e9, 1),
            # the same kernels back to back (their working set partly in the
            # 256 MB Infinity Cache)
            "plan_frac_hbm_warm": round(work["plan_bytes"] / t_plan_k / PEAK_HBM, 4),
            "combine_frac_hbm_warm": round(work["combine_bytes"] / t_copy / PEAK_HBM, 4),
            "scale_frac_hbm_warm": round(work["scale_bytes"] / t_scale_k / PEAK_HBM, 4),
            "combine_at_budget_GBs": round(work["combine_bytes"] / t_copy_budget / 1e9, 1),
            "combine_per_row_frac_hbm": round(work["combine_bytes"] / t_rows / PEAK_HBM, 4) if t_rows else None,
            "combine_per_row_frac_hbm_cold": (round(work["combine_bytes"] / t_rows_cold / PEAK_HBM, 4)
                                              if t_rows_cold else None),
            "device_copy_frac_hbm_cold": (round(work["combine_bytes"] / t_dev_copy_cold / PEAK_HBM, 4)
                                          if t_dev_copy_cold else None),
            "routed_rows_per_s": round(R / (ms * 1e-3), 1),
        },
        "overlap": {
            "consumer_tail_after_producer_us": None if tail is None else round(tail * 1e6, 2),
            "overlap_ratio": None if tail is None else round(max(0.0, min(1.0, 1.0 - tail / t_copy)), 4),
            "serial_ms_per_step": round(ms_serial, 4),
            "speedup_vs_serial": round(ms_serial / ms, 4),
        },
        "gathered_rows": None if ms_gathered is None else {
            "ms_per_step": round(ms_gathered, 4),
            "tokens_per_s": round(tokens_per_rank / (ms_gathered * 1e-3), 1),
            "plan_metadata_back_to_back_us": round(t_plan_meta * 1e6, 2),
        },
        "work": {k: v for k, v in work.items()},
    }
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, ids, w, x_recv, wgu, wd, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
