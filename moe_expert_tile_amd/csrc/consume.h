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
// in schedule order.  The standalone consumer kernel gives unit u to
// workgroup u mod n_cons.  In the overlapped down-GEMM launch the units are
// claimed from a counter in schedule order, by the launch's consumer
// workgroups and by producers that have run out of tiles (consume_claimed).
// A workgroup waits for a segment once, on its first unit of that segment.
// The wait is bounded: after `timeout` ticks of the 100 MHz constant clock it
// records MOE_ETIMEOUT in the plan's error word and every consumer workgroup
// leaves.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef unsigned int cv4u32 __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ int segment_of_unit(const int32_t* sunit, int n_rs, int seg, int u) {
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
__device__ __forceinline__ int wait_segment(const PlanLayout& L, int32_t* hdr, const int32_t* sfirst,
                                            const int32_t* snb, const uint32_t* __restrict__ flags, uint32_t epoch,
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

// Copy unit u of segment seg: bytes [lo, lo + kCopyChunk) of the segment,
// clipped to its end by the buffer bounds, every load before the first store.
// Returns the unit's bytes.
template <int NT>
__device__ __forceinline__ int64_t copy_unit(const PlanLayout& L, const int32_t* ssrc, const int32_t* sdst,
                                             const int32_t* sdoff, const int32_t* srows, const int32_t* sunit,
                                             const uint16_t* __restrict__ y, const RecvPtrs& recv, int seg, int u) {
  const int tid = threadIdx.x;
  const int64_t d = L.d;
  const int64_t bytes = (int64_t)srows[seg] * d * 2;
  const int64_t lo = (int64_t)(u - sunit[seg]) * kCopyChunk;
  const int64_t n = min((int64_t)kCopyChunk, bytes - lo);
  const __amdgpu_buffer_rsrc_t src = copy_rsrc((const char*)(y + (int64_t)ssrc[seg] * d) + lo, n);
  const __amdgpu_buffer_rsrc_t dst = copy_rsrc((char*)(recv.p[sdst[seg]] + (int64_t)sdoff[seg] * d) + lo, n);
  constexpr int VPT = kCopyChunk / (NT * 16);
  static_assert(VPT >= 1 && VPT * NT * 16 == kCopyChunk, "whole vectors per unit");
  cv4u32 v[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) v[k] = __builtin_amdgcn_raw_buffer_load_b128(src, (k * NT + tid) * 16, 0, kAgentLoad);
#pragma unroll
  for (int k = 0; k < VPT; ++k) __builtin_amdgcn_raw_buffer_store_b128(v[k], dst, (k * NT + tid) * 16, 0, kStreamStore);
  return n;
}

// One consumer workgroup of NT threads; `cid` in [0, n_cons), units assigned
// statically (standalone consumer kernel).  `s_go` is one int of the
// caller's LDS.
template <int NT>
__device__ void consume_segments(const PlanLayout& L, int32_t* ws, const uint16_t* __restrict__ y,
                                 const uint32_t* __restrict__ flags, uint32_t epoch, const RecvPtrs& recv,
                                 const CopyCtl& cc, int cid, int n_cons, int* s_go) {
  int32_t* hdr = ws + L.o_hdr;
  if (__hip_atomic_load(hdr + H_ERROR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  const int32_t* sfirst = ws + L.o_sfirst;
  const int32_t* snb = ws + L.o_snb;
  const int32_t* sdst = ws + L.o_sdst;
  const int32_t* sdoff = ws + L.o_sdoff;
  const int32_t* ssrc = ws + L.o_ssrc;
  const int32_t* srows = ws + L.o_srows;
  const int32_t* sunit = ws + L.o_sunit;
  // remote segments come first in schedule order; their units end where the
  // first local segment's begin
  const int n_rs = hdr[H_RSEGS];
  const int U = sunit[n_rs];
  if (cid >= U) return;
  int seg = 0, ready = -1;
  for (int u = cid; u < U; u += n_cons) {
    seg = segment_of_unit(sunit, n_rs, seg, u);
    if (seg != ready) {
      if (!wait_segment(L, hdr, sfirst, snb, flags, epoch, cc, ws, seg, s_go)) return;
      ready = seg;
    }
    const int64_t n = copy_unit<NT>(L, ssrc, sdst, sdoff, srows, sunit, y, recv, seg, u);
    pace_unit(cc, sdst[seg], n);
  }
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
  const int32_t* sfirst = ws + L.o_sfirst;
  const int32_t* snb = ws + L.o_snb;
  const int32_t* sdst = ws + L.o_sdst;
  const int32_t* sdoff = ws + L.o_sdoff;
  const int32_t* ssrc = ws + L.o_ssrc;
  const int32_t* srows = ws + L.o_srows;
  const int32_t* sunit = ws + L.o_sunit;
  const int n_rs = hdr[H_RSEGS];
  const int U = sunit[n_rs];
  const int cu = max(1, min(kClaimUnitsMax, U / (2 * (int)gridDim.x)));   // units per claim
  const int n_claims = (U + cu - 1) / cu;
  const int tid = threadIdx.x;
  if (tid == 0) s_word[1] = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int k = s_word[1];
  __syncthreads();
  int seg = 0, ready = -1;
  while (k < n_claims) {
    // the next claim is in flight while this one is copied
    if (tid == 0) s_word[1] = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int j = 0; j < cu; ++j) {
      const int u = k * cu + j;
      if (u < U) {
        seg = segment_of_unit(sunit, n_rs, seg, u);
        if (seg != ready) {
          if (!wait_segment(L, hdr, sfirst, snb, flags, epoch, cc, ws, seg, s_word)) return;
          ready = seg;
        }
        const int64_t n = copy_unit<NT>(L, ssrc, sdst, sdoff, srows, sunit, y, recv, seg, u);
        pace_unit(cc, sdst[seg], n);
      }
    }
    __syncthreads();
    k = s_word[1];
    __syncthreads();
  }
}

}  // namespace moe
