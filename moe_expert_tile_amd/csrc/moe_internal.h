// Internal definitions shared by the HIP kernels and the host orchestration
// of libmoe.so.  Nothing here is part of the public ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kMaxWorld = 64;
constexpr int kPairsPerBlock = 512;    // (token, slot) pairs per planner workgroup
constexpr int kPlanThreads = 256;
constexpr int kCopyChunk = 32768;      // bytes per consumer copy unit
constexpr int kGuBM = 256;             // gate/up GEMM tile rows
constexpr int kGuBN = 256;             // gate/up GEMM tile cols (128 gate + 128 up)
constexpr int kDnBN = 256;             // down GEMM tile cols
constexpr int kDnBM = 256;             // down GEMM tile rows: 256 compacted rows of one X_e, as gate/up's
// K steps of the GEMM configurations (gemm.hip asserts them); the host sizes
// the stream-K scratch with them
constexpr int kGuBK = 64;              // gate/up
constexpr int kDnBK = 64;              // down
constexpr int kMaxProducers = 256;     // persistent GEMM workgroups at most (one per CU on MI355X)
constexpr int kMinSkSteps = 16;        // shortest K range of a stream-K piece
// stream-K for a tail round only with tiles of at least this many K steps.
// Measured with the gate/up GEMM over compacted rows (same box, serial mode,
// threshold 128 -> 64): DeepSeek-like gate/up (112 steps, a tail round 19%
// full) 2485 -> 2392 us, Qwen3-like gate/up (64 steps, 33% full) 450 ->
// 432 us, Mixtral-like unchanged.  The short-K down GEMMs (24 and 32 steps)
// stay below it: there the partials' round trip costs as much as the tail
// round it removes.
constexpr int kMinSkKT = 64;
// ... but a GEMM whose tiles fill at most half of one round is split along
// K from 2 * kMinSkSteps steps on, so that each tile gets pieces of at most
// half its steps (decode's 120 gate/up tiles of 32 steps on 256 CUs:
// 59 -> 55 us; its 190 tiles at tb_M 64, three quarters of a round, went
// 62 -> 80 us).  With at least that many steps a piece never spans more
// than two tiles.
constexpr int kMinSkKTOneRound = 2 * kMinSkSteps;

// header words of the plan workspace (mirrors the public description)
enum Hdr {
  H_ERROR = 0, H_M = 1, H_BANDS = 2, H_REMOTE = 3, H_SEGS = 4, H_RSEGS = 5,
  H_GU_TILES = 6, H_DN_TILES = 7, H_UNITS = 8, H_RCOUNT = 9, H_GU_MT = 10, H_DN_MT = 11,
  // uint64 wall-clock stamps (100 MHz) raised by every producer / consumer
  // workgroup of the down-GEMM launch as it ends (atomic max, so no reset is
  // needed between calls): words 12-13 and 14-15
  H_T_PROD_END = 12, H_T_CONS_END = 14,
  H_DN_MT_R = 16,   // down row tiles holding remote rows (they come first)
  // overlapped down-GEMM launch: copy-unit claims handed out so far, and
  // producers that have started (the default Scratch::claim); both zeroed by
  // the gate/up launch, which precedes every down GEMM on the same stream
  H_CLAIM = 18, H_STARTED = 19,
  // planner: set by the plan builder once the group tables the pair placers
  // need are in memory; cleared by the counting launch that precedes it
  H_READY = 20,
  H_WORDS = 64
};

// Exact division of a non-negative int below 2^nbits by a fixed divisor d,
// with one 64-bit multiply and a shift: s = nbits + bit length of d, so
// 2^s > n d, and m = ceil(2^s / d); then floor(n m / 2^s) = floor(n / d),
// because n (m - 2^s / d) / 2^s < n / 2^s < 1 / d, and n / d is an integer
// or at least 1 / d below the next one.  m n < 2^(2 nbits + 1).
struct FastDiv {
  uint64_t m;
  int s, d;
};
inline FastDiv make_fastdiv(int d, int nbits) {
  int len = 0;
  while ((1 << len) <= d) ++len;
  FastDiv f;
  f.s = nbits + len;
  f.m = (((uint64_t)1 << f.s) + (uint64_t)d - 1) / (uint64_t)d;
  f.d = d;
  return f;
}
#if defined(__HIPCC__)
__host__ __device__
#endif
inline int fdiv(int n, const FastDiv& f) { return (int)(((uint64_t)(uint32_t)n * f.m) >> f.s); }

// Everything a kernel needs to find the plan arrays: sizes and int32 element
// offsets from the workspace base.  Built on the host, passed by value.
struct PlanLayout {
  int W, r, E_l, E, k, d, f, tb_m, mgb;
  int R, rows_cap, bands_cap, T_r, NB, NB_r, gu_mt_cap;
  int dn_ntn, dn_tpb;                  // down GEMM: column tiles, flag pairs per band (= column tiles)
  int gu_ntn;                          // gate/up GEMM n tiles (f / 128)
  int band_lds;                        // the plan builder keeps its per-band tables in LDS (else in btmp)
  FastDiv div_tb, div_mgb, div_wm1, div_hb, div_w, div_el;   // by tb_m, mgb, max(W - 1, 1), E_l + 2, W, E_l
  int sk_slots;                        // stream-K partial-sum slots (256x256 fp32 each) in the workspace
  int64_t o_hdr, o_c, o_low, o_grp, o_me, o_rowoff, o_rb, o_order, o_base;
  int64_t o_bexp, o_bdst, o_bsrc, o_bdoff, o_bval;
  int64_t o_sfirst, o_snb, o_sdst, o_sdoff, o_ssrc, o_srows, o_sunit;
  int64_t o_src, o_pos;
  int64_t o_bh, o_bhr;                 // per-block histograms (plan_count)
  int64_t o_obase;                     // [W + 1]: received rows from the owners before each owner
  int64_t o_grow, o_gcrow;             // [E_l][W]: first layout row and first compacted row of every group
  int64_t o_btmp;                      // [4 * (bands_cap + 1)]: the builder's per-band tables when not in LDS
  int64_t o_gband;                     // [E_l][W]: first band of every group in S
  int64_t o_gumt_row, o_gumt_exp;
  int64_t o_dnt_row, o_dnt_exp;
  // compacted rows (the layout without its padding rows, in layout order):
  // start of every expert, offset of every group inside its expert, first
  // compacted row of every band, and per compacted row its layout row and
  // its received row
  int64_t o_crowoff, o_ccum, o_bcrow, o_cmprow, o_cmpsrc;
  int64_t o_link;                      // uint64 [kMaxWorld] emulated link busy-until times
  int64_t o_gready;                    // uint64 [E_l * W] group-batched ready counters
  int64_t o_skc;                       // uint64 [2][kMaxProducers] stream-K tile counters (gate/up, down)
  int64_t o_skp;                       // float [sk_slots][256*256] stream-K partial sums
  int64_t total_words;
  int pair_off[kMaxWorld + 1];   // first (token, slot) pair of each owner
  int blk_off[kMaxWorld + 1];    // first planner block of each owner
  int tok_off[kMaxWorld + 1];    // first token of each owner
};

struct RecvPtrs {
  uint16_t* p[kMaxWorld];
};

// Scratch of moe_expert_combine's kernels: the stream-K partial sums and
// their epoch-tagged tile counters, and the two copy-claim counters of the
// overlapped down-GEMM launch (claims handed out, producers started).  By
// default they live in the plan workspace; the allocation-free entry point
// points them into a static device array instead.
struct Scratch {
  float* sk_part;       // [sk_slots][256*256] fp32
  uint64_t* sk_ctr;     // [2][kMaxProducers]: gate/up, down
  int32_t* claim;       // [2]: claims handed out, producers started
  uint64_t* link_free;  // [kMaxWorld]: emulated link of each destination busy until (1/1024 ticks, 100 MHz)
  uint64_t* gready;     // [kMaxGroups]: group-batched ready counters, epoch-tagged
  int sk_slots;
};
constexpr int kMaxGroups = 1024;       // E_l * W at most

// How the consumer waits and copies (moe_combine_opts):
//   signal 0: per-band tile flags, equal to the call's epoch when ready;
//   signal 1: one ready counter per (expert, destination) group, raised by
//             each down tile by the band heads and tails of the group it
//             holds and ready when it reads (epoch, 2 * bands * column tiles);
//   link_mbps > 0: every copy unit to owner o also takes bytes / rate on an
//             emulated link of owner o (reserved in order on the device
//             clock), and the copying workgroup waits until its transfer
//             would have ended.
struct CopyCtl {
  int64_t timeout;      // 100 MHz ticks
  uint32_t link_mbps;
  int signal;
  uint64_t* link_free;
  const uint64_t* gready;
};

// LDS carve-outs of the planner's second launch, in int words; the host
// sizes the launch's dynamic LDS with the same functions the kernel carves
// it with.  The builder keeps its expert x owner tables on chip and, when
// `bands` is set, four per-band tables of bands_cap + 1 words.
struct BuildLds {
  int c, grow, gcrow, base, gstart, low, bad, obase, me, ce, rowoff, crowoff, rb, order, gupre, dpre, sh, misc;
  int nx, ja, jb, on, total;
};
#if defined(__HIPCC__)
__host__ __device__
#endif
inline BuildLds build_lds(int W, int E_l, int bands_cap, bool bands) {
  BuildLds s;
  const int EW = E_l * W;
  int o = 0;
  s.c = o; o += EW;
  s.grow = o; o += EW;
  s.gcrow = o; o += EW;
  s.base = o; o += EW;
  s.gstart = o; o += EW + 1;
  s.low = o; o += W;
  s.bad = o; o += W;
  s.obase = o; o += W + 1;
  s.me = o; o += E_l;
  s.ce = o; o += E_l;
  s.rowoff = o; o += E_l + 1;
  s.crowoff = o; o += E_l + 1;
  s.rb = o; o += E_l;
  s.order = o; o += E_l;
  s.gupre = o; o += E_l + 1;
  s.dpre = o; o += 2 * (E_l + 1);
  s.sh = o; o += 32;
  s.misc = o; o += 8;
  const int nb = bands ? bands_cap + 1 : 0;
  s.nx = o; o += nb;    // segment started at the band: rows << 8 | bands, or 0
  s.ja = o; o += nb;    // the band's source row
  s.jb = o; o += nb;    // the band's receive offset
  s.on = o; o += nb;    // the band's owner
  s.total = o;
  return s;
}
// pair placers (workgroups 1.. of the second launch)
struct PlaceLds {
  int run, wc, run_g, wc_g, bp, pre_g, base_g, srow, scrow, pst, pct, sh, misc, total;
};
#if defined(__HIPCC__)
__host__ __device__
#endif
inline PlaceLds place_lds(int E_l, int E, int nw) {
  PlaceLds s;
  int o = 0;
  s.run = o; o += E_l + 1;
  s.wc = o; o += nw * (E_l + 1);
  s.run_g = o; o += E;
  s.wc_g = o; o += nw * E;
  s.bp = o; o += E_l;
  s.pre_g = o; o += E;
  s.base_g = o; o += E;
  s.srow = o; o += E_l;
  s.scrow = o; o += E_l;
  s.pst = o; o += kPlanThreads;   // padding runs of up to kPlanThreads groups: first row
  s.pct = o; o += kPlanThreads;   // ... and length
  s.sh = o; o += 32;
  s.misc = o; o += 8;
  s.total = o;
  return s;
}
constexpr int kBuildLdsBytes = 64 * 1024;   // cap on the planner's dynamic LDS (the default dynamic limit)

// host-side helpers (api.cpp)
bool make_layout(int W, int r, int E_l, int k, int d, int f, int tb_m, int mgb,
                 const int32_t* tokens, int64_t R, PlanLayout* L);
// moe_expert_combine; get_scratch == nullptr: the kernels' scratch is in the
// plan workspace, else get_scratch(device, &sc) supplies it (the counters are
// then cleared at the start of the call)
int combine_impl(const moe_shape* s, const void* plan_ws, const uint16_t* x_layout, const uint16_t* w_gate_up,
                 const uint16_t* w_down, uint16_t* h, uint16_t* y, uint32_t* flags, uint32_t epoch,
                 uint16_t* const* recv, const moe_combine_opts* opts, void* stream,
                 int (*get_scratch)(int dev, Scratch* out));

// launchers (defined next to their kernels); all asynchronous on `s`
hipError_t launch_plan(const PlanLayout& L, const int32_t* topk, const uint16_t* x_recv,
                       int32_t* ws, uint16_t* x_layout, hipStream_t s);
// gate/up GEMM: A rows from the layout `x` [rows_cap, d], or (gathered) from
// x_recv [R, d] through the plan's src_index
hipError_t launch_gateup(const PlanLayout& L, int32_t* ws, const Scratch& sc, const uint16_t* x, bool gathered,
                         const uint16_t* wgu, uint16_t* h, uint32_t epoch, int grid, hipStream_t s);
// down GEMM: `n_prod` persistent producer workgroups; the grid's remaining
// workgroups (if any) are consumers (consume.h).  Local bands are also
// written to recv.p[L.r].
hipError_t launch_down(const PlanLayout& L, int32_t* ws, const Scratch& sc, const uint16_t* h, const uint16_t* wd,
                       uint16_t* y, uint32_t* flags, uint32_t epoch, const RecvPtrs& recv, const CopyCtl& cc,
                       int n_prod, int grid, hipStream_t s);
// zeroes the counters of `sc` (tile counters, claim words, link times, group
// counters) with a fill kernel: the static scratch keeps the previous call's
// contents
hipError_t launch_clear_counters(const Scratch& sc, hipStream_t s);
hipError_t launch_consumer(const PlanLayout& L, int32_t* ws, const uint16_t* y,
                           const uint32_t* flags, uint32_t epoch, const RecvPtrs& recv,
                           const CopyCtl& cc, int grid, hipStream_t s);
// per-row ablation of the copy: one wavefront per remote row (COPY_ROWS mode)
hipError_t launch_consumer_rows(const PlanLayout& L, int32_t* ws, const uint16_t* y, const uint32_t* flags,
                                uint32_t epoch, const RecvPtrs& recv, int64_t timeout_ticks, hipStream_t s);
hipError_t launch_scale(const PlanLayout& L, const int32_t* ws, const uint16_t* recv_self,
                        const float* topk_w, uint16_t* out, hipStream_t s);

// device helpers ------------------------------------------------------------
#if defined(__HIPCC__)
__device__ __forceinline__ int32_t* ws_at(int32_t* ws, int64_t off) { return ws + off; }
__device__ __forceinline__ const int32_t* ws_at(const int32_t* ws, int64_t off) { return ws + off; }
#endif

}  // namespace moe
