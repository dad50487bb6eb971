// Consumer body: the second all-to-all of the tile-signal notes ("MoE 计算-通信
// 细粒度重叠：用 Tile 级信号把 All-to-All 藏在 GEMM 背后"), §3 Stage B, §5.2 and §5.3.
// Shared by the standalone consumer kernel and by the consumer workgroups of
// the overlapped down-GEMM launch.
//
// The remote segments are walked in schedule order: each waits until every
// tile flag of its bands equals this call's epoch (a band has a head and a
// tail flag per column tile: a row tile may end inside it), then its valid rows --
// contiguous in the layout and contiguous at the destination -- are copied
// into the owner's receive buffer.  The W owners are W buffers in HBM; the
// pages' one-sided remote put becomes a device-memory copy.  Local segments
// are not copied here: their rows never leave the rank, and the down GEMM's
// epilogue writes them straight into the rank's own receive buffer.
//
// Memory ordering: the producer stores a tile's rows at device scope (sc1,
// written through its XCD's L2), waits until every store is acknowledged and
// only then sets the tile's flags to epoch with relaxed agent-scope stores
// (no release fence).  Here wave 0 polls the flags with relaxed agent-scope
// loads; the tile's rows are read only after the flags were seen, with
// agent-scope (sc1) loads, 16 bytes per lane, which do not return lines this
// XCD cached earlier, so no acquire fence or cache-wide invalidation is
// issued and the producer's L2 contents on the same XCD survive.
//
// Work split: each segment is cut into units of kCopyChunk bytes, numbered
// in schedule order.  A workgroup keeps two units in flight: the next
// unit's loads go out before the current unit's stores.  The standalone consumer kernel gives unit u to
// workgroup u mod n_cons.  In the overlapped down-GEMM launch the units are
// claimed from a counter in schedule order, by the launch's consumer
// workgroups and by producers that have run out of tiles (consume_claimed).
// A workgroup waits for a segment once, on its first unit of that segment.
// The wait is bounded: after `timeout` ticks of the 100 MHz constant clock it
// records MOE_ETIMEOUT in the plan's error word and every consumer workgroup
// leaves.
#pragma once

#include <type_traits>

#include "moe_internal.h"

namespace moe {

typedef unsigned int cv4u32 __attribute__((ext_vector_type(4)));
// The plan's tables, written by the planner's launches and only read by the
// combine's kernels: loads through the constant address space with a
// wave-uniform index become scalar loads, which the vector memory counter
// does not track, so reading a table never waits for outstanding loads and
// stores (the GEMM's tile setup, the copy's next unit).
typedef const int32_t __attribute__((address_space(4))) ctab_t;

// Raw buffer resource over [base, base + bytes): accesses past the end read
// zero and drop their stores (gfx9-family word 3: 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t copy_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// cache-policy bit sc1 (bit 4): the same agent-scope load an agent-scope
// atomic load compiles to, so a line cached by this XCD before the
// producer's release is not returned stale
constexpr int kAgentLoad = 16;

// cache-policy bits of the copy's stores: nt (bit 1) and sc1 (bit 4), so the
// copied rows stream through without displacing the producers' operand lines
// from this XCD's L2 (same-box: the Qwen3- and DeepSeek-like overlapped down
// GEMMs ~1% faster, Mixtral-like unchanged)
constexpr int kStreamStore = 18;

#ifndef MOE_POLL_MAX_NAPS
#define MOE_POLL_MAX_NAPS 32   // longest pause between flag polls, in units of 128 clocks
#endif

// Segment of copy unit u, searching forward from `seg` (units only grow):
// a few steps ahead, then a binary search over the rest.
template <class P>
__device__ __forceinline__ int segment_of_unit(P sunit, int n_rs, int seg, int u) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (sunit[seg + 1] > u) return seg;
    ++seg;
  }
  int lo = seg, hi = n_rs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sunit[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Wave 0 waits until segment `seg` is ready: both tile flags (band head and
// band tail) of its bands for every column tile equal `epoch` (signal 0), or
// its group's ready counter reads (epoch, 2 * bands of the group * column
// tiles) (signal 1).  Bounded by `timeout`
// ticks of the 100 MHz clock; on timeout the plan's error word becomes
// MOE_ETIMEOUT.  Returns 0 if the workgroup must stop.  Every thread of the
// workgroup calls it.
template <class P>
__device__ __forceinline__ int wait_segment(const PlanLayout& L, int32_t* hdr, P sfirst,
                                            P snb, const uint32_t* __restrict__ flags, uint32_t epoch,
                                            const CopyCtl& cc, const int32_t* ws, int seg, int* s_go) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int tpb = L.dn_tpb;
  if (tid < 64) {
    // flag words [2 tpb b, 2 tpb (b + 1)) belong to band b
    const int f0 = 2 * sfirst[seg] * tpb, f1 = 2 * (sfirst[seg] + snb[seg]) * tpb;
    int gi = 0;
    uint64_t want = 0;
    if (cc.signal) {
      // the segment's group: (expert of its first band, its destination)
      const int e = ws[L.o_bexp + sfirst[seg]], o = ws[L.o_sdst + seg];
      const int n = ws[L.o_c + e * L.W + o];
      gi = e * L.W + o;
      want = ((uint64_t)epoch << 32) | (uint32_t)(2 * ((n + L.tb_m - 1) / L.tb_m) * tpb);
    }
    const uint64_t t0 = wall_clock64();
    int go = 1;
    // exponential back-off between polls (128 clocks doubling to ~4K), and
    // the clock and the shared error word read only every 16th poll: many
    // waiting workgroups polling a few cache lines slow the producers down
    int naps = 1;
    for (int poll = 1;; ++poll) {
      bool ok = true;
      if (cc.signal) {
        ok = __hip_atomic_load(cc.gready + gi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want;
      } else {
        for (int i = f0 + lane; i < f1; i += 64)
          ok &= (__hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch);
      }
      if (__ballot(!ok) == 0) break;
      if ((poll & 15) == 0) {
        if ((int64_t)(wall_clock64() - t0) > cc.timeout) {
          if (lane == 0)
            __hip_atomic_store(hdr + H_ERROR, 4 /* MOE_ETIMEOUT */, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          go = 0;
          break;
        }
        if (__hip_atomic_load(hdr + H_ERROR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
          go = 0;
          break;
        }
      }
      for (int z = 0; z < naps; ++z) __builtin_amdgcn_s_sleep(2);
      naps = min(2 * naps, MOE_POLL_MAX_NAPS);
    }
    if (lane == 0) *s_go = go;
  }
  __syncthreads();
  const int go = *s_go;
  __syncthreads();
  return go;
}

// Emulated link of destination `dst` (cc.link_mbps > 0): the unit's bytes
// take bytes / rate on it, in a slot that starts no earlier than the unit's
// arrival.  The link's busy-until time L (1/1024 tick of the 100 MHz clock)
// only grows: the unit first raises it to its arrival time (atomic max),
// then takes [L, L + dur) with an atomic add.  Slots handed out by the adds
// never overlap, a max in between only opens an idle gap, and neither step
// retries: a compare-and-swap loop measured ~20x slower, with hundreds of
// workgroups retrying one device-scope word at one memory-side round trip
// per attempt.  The workgroup waits until its slot ends.  Every thread of
// the workgroup calls it.
__device__ __forceinline__ void pace_unit(const CopyCtl& cc, int dst, int64_t bytes) {
  if (cc.link_mbps == 0) return;
  if (threadIdx.x == 0) {
    const uint64_t dur = (uint64_t)bytes * 102400u / cc.link_mbps;   // 100 ticks per us, x1024
    uint64_t* link = cc.link_free + dst;
    __hip_atomic_fetch_max(link, (uint64_t)wall_clock64() << 10, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t end = __hip_atomic_fetch_add(link, dur, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + dur;
    while ((wall_clock64() << 10) < end) __builtin_amdgcn_s_sleep(1);
  }
  __syncthreads();
}

// One copy unit in flight: its bytes in registers (VPT 16-byte vectors per
// thread), where they go, how many there are and the destination rank.
template <int NT>
struct CopyUnit {
  static constexpr int VPT = kCopyChunk / (NT * 16);
  static_assert(VPT >= 1 && VPT * NT * 16 == kCopyChunk, "whole vectors per unit");
  cv4u32 v[VPT];
  char* to;
  int64_t n;
  int dst;   // -1: no unit
};

// The segment tables the copy reads, through P: the constant address space
// (const ctab_t*, scalar loads) where a workgroup copies many units with
// loads and stores in flight, so that reading a table does not wait for
// them; plain pointers (vector loads) where each workgroup copies one unit:
// with thousands of such workgroups the scalar loads measured 7% slower.
template <class P>
struct SegTabs {
  P sfirst, snb, sdst, sdoff, ssrc, srows, sunit;
};
template <class P>
__device__ __forceinline__ SegTabs<P> seg_tabs(const PlanLayout& L, const int32_t* ws) {
  const P t = (P)ws;
  return SegTabs<P>{t + L.o_sfirst, t + L.o_snb, t + L.o_sdst, t + L.o_sdoff, t + L.o_ssrc, t + L.o_srows, t + L.o_sunit};
}
template <bool PIPE>
using SegPtr = typename std::conditional<PIPE, const ctab_t*, const int32_t*>::type;

// Load unit u of segment seg: bytes [lo, lo + kCopyChunk) of the segment,
// clipped to its end by the buffer bounds, read at device scope.
template <int NT, class P>
__device__ __forceinline__ void load_unit(const PlanLayout& L, const SegTabs<P>& T, const uint16_t* __restrict__ y,
                                          const RecvPtrs& recv, int seg, int u, CopyUnit<NT>& U) {
  const int tid = threadIdx.x;
  const int64_t d = L.d;
  const int64_t bytes = (int64_t)T.srows[seg] * d * 2;
  const int64_t lo = (int64_t)(u - T.sunit[seg]) * kCopyChunk;
  const int64_t n = min((int64_t)kCopyChunk, bytes - lo);
  const __amdgpu_buffer_rsrc_t src = copy_rsrc((const char*)(y + (int64_t)T.ssrc[seg] * d) + lo, n);
  U.dst = T.sdst[seg];
  U.to = (char*)(recv.p[U.dst] + (int64_t)T.sdoff[seg] * d) + lo;
  U.n = n;
#pragma unroll
  for (int k = 0; k < CopyUnit<NT>::VPT; ++k)
    U.v[k] = __builtin_amdgcn_raw_buffer_load_b128(src, (k * NT + tid) * 16, 0, kAgentLoad);
}

// Store a loaded unit, then take its slot on the destination's emulated
// link (if any).
template <int NT>
__device__ __forceinline__ void store_unit(const CopyCtl& cc, const CopyUnit<NT>& U) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t dst = copy_rsrc(U.to, U.n);
#pragma unroll
  for (int k = 0; k < CopyUnit<NT>::VPT; ++k)
    __builtin_amdgcn_raw_buffer_store_b128(U.v[k], dst, (k * NT + tid) * 16, 0, kStreamStore);
  pace_unit(cc, U.dst, U.n);
}

// The copy loop of one workgroup.  PIPE: software-pipelined over two units
// in flight -- unit j's loads go out before unit j-1's stores, and the two
// units alternate between two register sets (A, B), so no unit's data is
// moved between registers; for a few workgroups with many units each.
// Without PIPE each unit is stored before the next is loaded, with half the
// registers, so more workgroups fit a CU: for grids of one unit per
// workgroup.  next() gives the workgroup's next unit (-1 when done; it may
// wait, and must be called by every thread).  Returns 0 if the workgroup
// must stop (timeout or error).
template <int NT, bool PIPE, class Next>
__device__ __forceinline__ int copy_units(const PlanLayout& L, int32_t* hdr, const int32_t* ws,
                                          const SegTabs<SegPtr<PIPE>>& T,
                                          const uint16_t* __restrict__ y, const uint32_t* __restrict__ flags,
                                          uint32_t epoch, const RecvPtrs& recv, const CopyCtl& cc, int n_rs,
                                          int* s_go, Next next) {
  int seg = 0, ready = -1;
  CopyUnit<NT> A, B;
  A.dst = -1;
  B.dst = -1;
  // find unit u's segment, waiting for it if it is not the one already
  // waited for
  auto enter = [&](int u) __attribute__((always_inline)) {
    seg = __builtin_amdgcn_readfirstlane(segment_of_unit(T.sunit, n_rs, seg, u));
    if (seg != ready) {
      if (!wait_segment(L, hdr, T.sfirst, T.snb, flags, epoch, cc, ws, seg, s_go)) return false;
      ready = seg;
    }
    return true;
  };
  for (;;) {
    int u = next();
    if (u < 0) break;
    if (!enter(u)) return 0;
    load_unit<NT>(L, T, y, recv, seg, u, A);
    if (!PIPE) {
      store_unit<NT>(cc, A);
      A.dst = -1;
      continue;
    }
    if (B.dst >= 0) store_unit<NT>(cc, B);
    B.dst = -1;
    u = next();
    if (u < 0) break;
    if (!enter(u)) return 0;
    load_unit<NT>(L, T, y, recv, seg, u, B);
    store_unit<NT>(cc, A);
    A.dst = -1;
  }
  if (A.dst >= 0) store_unit<NT>(cc, A);
  if (B.dst >= 0) store_unit<NT>(cc, B);
  return 1;
}

// One consumer workgroup of NT threads; `cid` in [0, n_cons), units assigned
// statically (standalone consumer kernel).  `s_go` is one int of the
// caller's LDS.
template <int NT, bool PIPE>
__device__ void consume_segments(const PlanLayout& L, int32_t* ws, const uint16_t* __restrict__ y,
                                 const uint32_t* __restrict__ flags, uint32_t epoch, const RecvPtrs& recv,
                                 const CopyCtl& cc, int cid, int n_cons, int* s_go) {
  int32_t* hdr = ws + L.o_hdr;
  if (__hip_atomic_load(hdr + H_ERROR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  const SegTabs<SegPtr<PIPE>> T = seg_tabs<SegPtr<PIPE>>(L, ws);
  // remote segments come first in schedule order; their units end where the
  // first local segment's begin
  const int n_rs = hdr[H_RSEGS];
  const int U = T.sunit[n_rs];
  int u = cid - n_cons;
  copy_units<NT, PIPE>(L, hdr, ws, T, y, flags, epoch, recv, cc, n_rs, s_go, [&]() __attribute__((always_inline)) {
    u += n_cons;
    return u < U ? u : -1;
  });
}

// Consumer with claimed work, for the overlapped down-GEMM launch: the
// remote copy units are handed out kClaimUnits at a time, in schedule order,
// from the counter claim[0] (zeroed by the gate/up launch before it).
// The launch's consumer workgroups run it from the start; producers that
// have run out of tiles join them, so the dedicated consumer can be small
// and the copies left when the last tiles finish are shared by every CU.
// Each workgroup asks for its next claim while it copies the current one.
// A claim is U / (2 x the launch's workgroups) units, between 1 and 8: on
// large layers 8-unit claims (256 KB) made the overlapped down GEMM
// 0.7-1.6% faster than 2-unit ones (fewer atomics on one word while it
// runs), but a decode-size layer has only ~130 units, and a few long claims
// copied one unit after another left a 25 us tail after the last producer.
// `s_word` is two ints of the caller's LDS.
constexpr int kClaimUnitsMax = 8;

template <int NT>
__device__ void consume_claimed(const PlanLayout& L, int32_t* ws, int32_t* claim, const uint16_t* __restrict__ y,
                                const uint32_t* __restrict__ flags, uint32_t epoch, const RecvPtrs& recv,
                                const CopyCtl& cc, int* s_word) {
  int32_t* hdr = ws + L.o_hdr;
  if (__hip_atomic_load(hdr + H_ERROR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  const SegTabs<SegPtr<true>> T = seg_tabs<SegPtr<true>>(L, ws);
  const int n_rs = hdr[H_RSEGS];
  const int U = T.sunit[n_rs];
  const int cu = max(1, min(kClaimUnitsMax, U / (2 * (int)gridDim.x)));   // units per claim
  const int n_claims = (U + cu - 1) / cu;
  const int tid = threadIdx.x;
  // the claim being copied (k) and the next one, asked for while k is
  // copied; j: the next unit of claim k
  int k = -1, j = cu;
  if (tid == 0) s_word[1] = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  copy_units<NT, true>(L, hdr, ws, T, y, flags, epoch, recv, cc, n_rs, s_word, [&]() __attribute__((always_inline)) {
    for (;;) {
      if (j < cu) {
        const int u = k * cu + j++;
        if (u < U) return u;
      }
      __syncthreads();
      k = __builtin_amdgcn_readfirstlane(s_word[1]);
      __syncthreads();
      if (k >= n_claims) return -1;
      if (tid == 0) s_word[1] = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      j = 0;
    }
  });
}

}  // namespace moe
