// Planner: Stage A of the tile-signal notes ("MoE 计算-通信细粒度重叠：用 Tile 级信号把
// All-to-All 藏在 GEMM 背后", §3 and §4.2-§4.5, segments §5.2), on the device.
//
//   K1 plan_count   one workgroup per 512 (token, slot) pairs of one owner:
//                   LDS histograms of the local experts, of "below this rank's
//                   experts" (for receive offsets) and, for the rank's own
//                   tokens, of all experts (for the owner-side slot table).
//   K2 plan_build_place, one launch of 1 + NB workgroups:
//     workgroup 0, the builder: sums the histograms into group counts, lays
//                   out the groups (padded offsets in X_e, compacted offsets,
//                   expert starts), hands those few tables to the placers and
//                   raises a ready word, then builds the rule (ii) expert
//                   order, the band list S (remote bands first), the combine
//                   plan, segments and their copy units, and the GEMMs'
//                   row-tile tables -- every step a parallel pass or a scan.
//     workgroups 1..NB, the placers, one per pair block: prefixes of their
//                   own from the histograms, then (once the builder's tables
//                   are ready) the stable rank of every pair inside its
//                   (expert, owner) group with bit-sliced wave ballots + LDS
//                   carries -> src_index of every real layout row, the
//                   compacted-row tables, and the owner-side slot of each of
//                   the rank's own pairs; they also write the padding entries
//                   (-1) of src_index.
//   K4 plan_gather  one wavefront per layout row: X[row] = x_recv[src] or 0,
//                   16-byte coalesced loads and stores.
//
// Stability: pairs are visited in (owner, token, slot) order — blocks in
// order, rounds of 256 pairs in order, wavefronts in order, lanes in order —
// so every rank computed here is the rank in arrival order.
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Inclusive scan over the 64 lanes of a wavefront with DPP row shifts (scan
// within each row of 16 lanes) and row broadcasts (lane 15 into the next row,
// lane 31 into rows 2 and 3); disabled or out-of-row source lanes add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 (rows 1, 3)
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 (rows 2, 3)
  return x;
}

// Exclusive scan of a pair of ints per thread over the workgroup of
// kPlanThreads threads: wavefront scans, then every thread adds the totals
// of the wavefronts below its own (read in parallel from LDS).  `sh` holds
// 2 ints per wavefront.  Two barriers; `sh` is free again on return.
__device__ int2 block_scan2(int a, int b, int* sh, int2* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int nw = kPlanThreads / 64;
  const int xa = wave_incl_scan(a), xb = wave_incl_scan(b);
  if (lane == 63) {
    sh[2 * w] = xa;
    sh[2 * w + 1] = xb;
  }
  __syncthreads();
  int pa = 0, pb = 0, ta = 0, tb = 0;
  for (int i = 0; i < nw; ++i) {
    const int u = sh[2 * i], v = sh[2 * i + 1];
    ta += u;
    tb += v;
    if (i < w) {
      pa += u;
      pb += v;
    }
  }
  __syncthreads();
  *total = make_int2(ta, tb);
  return make_int2(pa + xa - a, pb + xb - b);
}

__device__ __forceinline__ int block_scan(int v, int* sh, int* total) {
  int2 t;
  const int2 p = block_scan2(v, 0, sh, &t);
  *total = t.x;
  return p.x;
}

// Exclusive scan over n items: val(i) gives item i, out(i, prefix) receives
// its exclusive prefix.  Items are split into contiguous per-thread chunks;
// val(i) is read before out(i) is called, so the scan may work in place.
// Ends with a barrier: out's LDS writes are visible on return.
template <class F, class G>
__device__ int scan_items(int n, F val, G out, int* sh) {
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += val(i);
  int total;
  int run = block_scan(local, sh, &total);
  for (int i = lo; i < hi; ++i) { const int v = val(i); out(i, run); run += v; }
  __syncthreads();
  return total;
}

// The same over pairs: val(i) returns int2 (x, y), out(i, prefix) receives
// the exclusive int2 prefix.  Returns the int2 totals.
template <class F, class G>
__device__ int2 scan_items2(int n, F val, G out, int* sh) {
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int la = 0, lb = 0;
  for (int i = lo; i < hi; ++i) {
    const int2 v = val(i);
    la += v.x;
    lb += v.y;
  }
  int2 total;
  int2 run = block_scan2(la, lb, sh, &total);
  for (int i = lo; i < hi; ++i) {
    const int2 v = val(i);
    out(i, run);
    run.x += v.x;
    run.y += v.y;
  }
  __syncthreads();
  return total;
}

// Largest i in [0, n) with a[i] <= x (a ascending, a[0] <= x).
__device__ __forceinline__ int upper_index(const int* a, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int owner_of_block(const PlanLayout& L, int b) {
  int o = 0;
  while (o < L.W - 1 && b >= L.blk_off[o + 1]) ++o;
  return o;
}

// Relaxed agent-scope (device-wide) accesses to the words the builder hands
// to the placers: the stores write through this XCD's L2 to the memory side
// and the loads do not return lines another XCD's L2 cached earlier.
__device__ __forceinline__ void agent_store(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int agent_load(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Sum of a[b * stride + x] over b in [b0, b1), 16 independent loads in
// flight per thread.
__device__ __forceinline__ int sum_blocks(const int32_t* __restrict__ a, int64_t stride, int x, int b0, int b1) {
  int s = 0;
  for (int b = b0; b < b1; b += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = (b + u < b1) ? a[(int64_t)(b + u) * stride + x] : 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) s += v[u];
  }
  return s;
}

__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(PlanLayout L, const int32_t* __restrict__ topk,
                                                                 int32_t* __restrict__ ws) {
  extern __shared__ int sh[];
  const int b = blockIdx.x;
  const int o = owner_of_block(L, b);
  const int p0 = L.pair_off[o] + (b - L.blk_off[o]) * kPairsPerBlock;
  const int p1 = min(p0 + kPairsPerBlock, L.pair_off[o + 1]);
  const bool own = (o == L.r);
  const int nb = L.E_l + 2 + (own ? L.E : 0);
  // the next launch's placers wait for the builder to raise this word
  if (b == 0 && threadIdx.x == 0) agent_store(ws + L.o_hdr + H_READY, 0);
  for (int i = threadIdx.x; i < nb; i += blockDim.x) sh[i] = 0;
  __syncthreads();
  const int lo = L.r * L.E_l;
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int g = topk[p];
    if (g < 0 || g >= L.E) {
      atomicAdd(&sh[L.E_l + 1], 1);
      continue;
    }
    const int e = g - lo;
    if (e >= 0 && e < L.E_l) atomicAdd(&sh[e], 1);
    else if (g < lo) atomicAdd(&sh[L.E_l], 1);
    if (own) atomicAdd(&sh[L.E_l + 2 + g], 1);
  }
  __syncthreads();
  int32_t* bh = ws + L.o_bh + (int64_t)b * (L.E_l + 2);
  for (int i = threadIdx.x; i < L.E_l + 2; i += blockDim.x) bh[i] = sh[i];
  if (own) {
    int32_t* bhr = ws + L.o_bhr + (int64_t)(b - L.blk_off[L.r]) * L.E;
    for (int g = threadIdx.x; g < L.E; g += blockDim.x) bhr[g] = sh[L.E_l + 2 + g];
  }
}

// The plan builder (workgroup 0 of the second launch).  kBandLds: its
// per-band tables live in LDS, else in the workspace's btmp region.
template <bool kBandLds>
__device__ void build_plan(const PlanLayout& L, int32_t* __restrict__ ws) {
  extern __shared__ int smem[];
  const int tid = threadIdx.x;
  constexpr int nt = kPlanThreads;
  const int W = L.W, r = L.r, E_l = L.E_l, tb = L.tb_m;
  const int HB = E_l + 2;
  const int EW = E_l * W;
  const BuildLds S = build_lds(W, E_l, L.bands_cap, kBandLds);
  int32_t* hdr = ws + L.o_hdr;
  int* c = smem + S.c;             // [E_l][W] group sizes
  int* grow = smem + S.grow;       // [E_l][W] first layout row of every group
  int* gcrow = smem + S.gcrow;     // [E_l][W] first compacted row of every group
  int* base = smem + S.base;       // [W][E_l] receive-buffer bases
  int* gstart = smem + S.gstart;   // [E_l*W + 1] first band of every group in S order
  int* low = smem + S.low;         // [W] pairs of owner o with an expert below this rank's
  int* bad = smem + S.bad;         // [W] expert ids out of range, per owner
  int* obase = smem + S.obase;     // [W + 1] received rows from the owners before o
  int* me = smem + S.me;           // [E_l] rows of X_e
  int* ce = smem + S.ce;           // [E_l] real rows of X_e
  int* rowoff = smem + S.rowoff;   // [E_l + 1]
  int* crowoff = smem + S.crowoff; // [E_l + 1] first compacted row of X_e
  int* rb = smem + S.rb;           // [E_l] remote bands of every expert
  int* order = smem + S.order;     // [E_l] rule (ii) order
  int* gupre = smem + S.gupre;     // [E_l + 1] gate/up row tiles before each expert (rule (ii) order)
  int* sh = smem + S.sh;           // scan scratch
  int* misc = smem + S.misc;
  const int32_t* __restrict__ bh = ws + L.o_bh;

  // (a) group counts c[e][o], low[o] and bad ids per owner: one thread per
  //     (owner, histogram column), summing the owner's blocks with up to 16
  //     loads in flight
  for (int it = tid; it < W * HB; it += nt) {
    const int o = fdiv(it, L.div_hb), x = it - o * HB;
    const int s = sum_blocks(bh, HB, x, L.blk_off[o], L.blk_off[o + 1]);
    if (x < E_l) c[x * W + o] = s;
    else if (x == E_l) low[o] = s;
    else bad[o] = s;
  }
  __syncthreads();
  int lr = 0, lb = 0;
  for (int i = tid; i < EW; i += nt) lr += c[i];
  for (int o = tid; o < W; o += nt) lb += bad[o];
  int2 tot;
  (void)block_scan2(lr, lb, sh, &tot);
  const int rcount = tot.x, bad_total = tot.y;
  if (bad_total > 0 || rcount != L.R) {
    if (tid == 0) {
      for (int i = 1; i < H_WORDS; ++i)
        if (i != H_READY) hdr[i] = 0;
      hdr[H_RCOUNT] = rcount;
      agent_store(hdr + H_ERROR, 5);  // MOE_EROUTING
      wait_stores();
      agent_store(hdr + H_READY, 1);  // the placers see the error and leave
    }
    return;
  }

  // (b) the layout.  One pair scan over the groups in (expert, owner order)
  //     order -- remote owners ascending, then r -- gives every group's
  //     first row in X (remote groups padded to whole bands) and its first
  //     compacted row; one scan over (owner, expert) order gives the
  //     receive-buffer bases (owner o's pairs below global expert r*E_l + e)
  //     and the received rows from the owners before each owner.
  auto owner_at = [&](int q) { return (q < W - 1) ? (q < r ? q : q + 1) : r; };
  const int2 xtot = scan_items2(
      EW,
      [&](int i) {
        const int e = fdiv(i, L.div_w), o = owner_at(i - e * W);
        const int n = c[e * W + o];
        return make_int2(o == r ? n : fdiv(n + tb - 1, L.div_tb) * tb, n);
      },
      [&](int i, int2 pre) {
        const int e = fdiv(i, L.div_w), o = owner_at(i - e * W);
        grow[e * W + o] = pre.x;
        gcrow[e * W + o] = pre.y;
      },
      sh);
  (void)scan_items(
      EW,
      [&](int i) {
        const int o = fdiv(i, L.div_el), e = i - o * E_l;
        return c[e * W + o];
      },
      [&](int i, int pre) { base[i] = pre; }, sh);
  // expert starts, sizes, remote bands; owner bases; receive bases relative
  // to each owner
  for (int e = tid; e < E_l; e += nt) {
    const int q0 = owner_at(0);
    rowoff[e] = grow[e * W + q0];
    crowoff[e] = gcrow[e * W + q0];
    const int end = e + 1 < E_l ? grow[(e + 1) * W + q0] : xtot.x;
    const int cend = e + 1 < E_l ? gcrow[(e + 1) * W + q0] : xtot.y;
    me[e] = end - rowoff[e];
    ce[e] = cend - crowoff[e];
    rb[e] = fdiv(me[e] - c[e * W + r], L.div_tb);   // remote groups are whole bands
  }
  for (int o = tid; o <= W; o += nt) obase[o] = o < W ? base[o * E_l] : rcount;
  if (tid == 0) {
    rowoff[E_l] = xtot.x;
    crowoff[E_l] = xtot.y;   // = rcount
  }
  __syncthreads();
  for (int i = tid; i < EW; i += nt) {
    const int o = fdiv(i, L.div_el);
    base[i] += low[o] - obase[o];
  }
  const int M = xtot.x;
  // rule (ii) order: more remote bands first, ties to the lower id
  for (int e = tid; e < E_l; e += nt) {
    int rank = 0;
    const int mine = rb[e];
    for (int x = 0; x < E_l; ++x) {
      const int v = rb[x];
      rank += (v > mine) || (v == mine && x < e);
    }
    order[rank] = e;
  }

  // (c) hand the placers what they need -- group sizes, first layout and
  //     compacted rows of every group, owner receive bases -- with
  //     device-scope stores, wait for them, then raise the ready word
  for (int i = tid; i < EW; i += nt) {
    agent_store(ws + L.o_c + i, c[i]);
    agent_store(ws + L.o_grow + i, grow[i]);
    agent_store(ws + L.o_gcrow + i, gcrow[i]);
  }
  for (int i = tid; i <= W; i += nt) agent_store(ws + L.o_obase + i, obase[i]);
  if (tid == 0) agent_store(hdr + H_ERROR, 0);
  wait_stores();
  __syncthreads();
  if (tid == 0) agent_store(hdr + H_READY, 1);

  // the rest is read by the GEMMs, the consumer and the scale, all later
  // launches, and by inspection
  for (int i = tid; i < EW; i += nt) {
    const int e = fdiv(i, L.div_w);
    ws[L.o_base + i] = base[i];
    ws[L.o_grp + i] = grow[i] - rowoff[e];     // offsets inside X_e
    ws[L.o_ccum + i] = gcrow[i] - crowoff[e];
  }
  for (int i = tid; i < W; i += nt) ws[L.o_low + i] = low[i];
  for (int i = tid; i <= E_l; i += nt) {
    ws[L.o_rowoff + i] = rowoff[i];
    ws[L.o_crowoff + i] = crowoff[i];
  }
  for (int i = tid; i < E_l; i += nt) {
    ws[L.o_me + i] = me[i];
    ws[L.o_rb + i] = rb[i];
    ws[L.o_order + i] = order[i];
  }

  // (d) groups in schedule order: remote groups of experts in rule (ii)
  //     order (owners ascending, r skipped), then the local group of every
  //     expert
  const int NGR = E_l * (W - 1);
  const int NG = E_l * W;
  auto group_eo = [&](int gi, int& e, int& o) {
    if (gi < NGR) {
      const int qe = fdiv(gi, L.div_wm1);
      e = order[qe];
      const int q = gi - qe * (W - 1);
      o = q < r ? q : q + 1;
    } else {
      e = gi - NGR;
      o = r;
    }
  };
  const int B = scan_items(
      NG,
      [&](int gi) {
        int e, o;
        group_eo(gi, e, o);
        return fdiv(c[e * W + o] + tb - 1, L.div_tb);
      },
      [&](int gi, int pre) { gstart[gi] = pre; }, sh);
  if (B > L.bands_cap) {
    if (tid == 0) {
      for (int i = 1; i < H_WORDS; ++i)
        if (i != H_READY) hdr[i] = 0;
      hdr[H_ERROR] = 2;
    }
    return;
  }
  const int n_remote = NGR < NG ? gstart[NGR] : B;
  if (tid == 0) gstart[NG] = B;
  // every group's first band in S, for the down GEMM's epilogue
  for (int gi = tid; gi < NG; gi += nt) {
    int e, o;
    group_eo(gi, e, o);
    ws[L.o_gband + e * W + o] = gstart[gi];
  }

  // per-band tables of the segment scan
  int* nx;   // [B] segment started at the band: rows << 8 | bands, or 0
  int* ja;   // [B] source row
  int* jb;   // [B] receive offset
  int* on;   // [B] owner
  if constexpr (kBandLds) {
    nx = smem + S.nx; ja = smem + S.ja; jb = smem + S.jb; on = smem + S.on;
  } else {
    int* t = ws + L.o_btmp;
    const int nb = L.bands_cap + 1;
    nx = t; ja = t + nb; jb = t + 2 * nb; on = t + 3 * nb;
  }

  // (e) bands in S order, one thread per band.  Each band also decides
  //     whether it starts a segment (§5.2): the first and the last remote
  //     band alone; otherwise runs of <= mgb bands that restart at every
  //     group boundary (so a segment never crosses a group and is read off
  //     the band's own group).  A starting band keeps its segment's bands
  //     and rows for the scan below, which numbers the segments and places
  //     their copy units; the band tables nx, ja, jb, on hold the segment,
  //     source row, receive offset and owner.
  int32_t* bexp = ws + L.o_bexp;
  int32_t* bdst = ws + L.o_bdst;
  int32_t* bsrc = ws + L.o_bsrc;
  int32_t* bdoff = ws + L.o_bdoff;
  int32_t* bval = ws + L.o_bval;
  int32_t* bcrow = ws + L.o_bcrow;
  const int mgb = L.mgb;
  __syncthreads();   // gstart complete
  for (int b = tid; b < B; b += nt) {
    const int gi = upper_index(gstart, NG, b);   // the non-empty group holding band b
    int e, o;
    group_eo(gi, e, o);
    const int gs = gstart[gi];
    const int ge = gstart[gi + 1];
    const int q = b - gs;
    const int n = c[e * W + o];
    const int v = min(tb, n - q * tb);
    const int src_row = grow[e * W + o] + q * tb;
    const int dst_off = base[o * E_l + e] + q * tb;
    bexp[b] = e;
    bdst[b] = o;
    bsrc[b] = src_row;
    bdoff[b] = dst_off;
    bval[b] = v;
    bcrow[b] = gcrow[e * W + o] + q * tb;
    // segment start and the first band after the segment
    bool st;
    int nxt;
    if (gi < NGR) {
      const int off = b - (gs > 1 ? gs : 1);   // -1 only for band 0, which is alone
      const int m = off >= 0 ? off - fdiv(off, L.div_mgb) * mgb : 0;
      st = q == 0 || b == n_remote - 1 || (off >= 0 && m == 0);
      nxt = off >= 0 ? b + mgb - m : b + 1;
      if (b < n_remote - 1) nxt = min(nxt, n_remote - 1);
      else nxt = b + 1;
    } else {
      const int m = q - fdiv(q, L.div_mgb) * mgb;
      st = m == 0;
      nxt = b + mgb - m;
    }
    nxt = min(nxt, ge);
    const int nb = nxt - b;
    nx[b] = st ? ((min(nb * tb, n - q * tb) << 8) | nb) : 0;   // rows << 8 | bands (<= 64)
    ja[b] = src_row;
    jb[b] = dst_off;
    on[b] = o;
  }
  int32_t* sfirst = ws + L.o_sfirst;
  int32_t* snb = ws + L.o_snb;
  int32_t* sdst = ws + L.o_sdst;
  int32_t* sdoff = ws + L.o_sdoff;
  int32_t* ssrc = ws + L.o_ssrc;
  int32_t* srows = ws + L.o_srows;
  int32_t* sunit = ws + L.o_sunit;
  const int64_t row_bytes = (int64_t)L.d * 2;
  auto units_of = [&](int rows) { return (int)((rows * row_bytes + kCopyChunk - 1) / kCopyChunk); };
  if (tid == 0) misc[0] = -1;
  __syncthreads();
  const int2 stot = scan_items2(
      B,
      [&](int b) {
        const int sg = nx[b];
        return sg ? make_int2(1, units_of(sg >> 8)) : make_int2(0, 0);
      },
      [&](int b, int2 pre) {
        const int sg = nx[b];
        if (!sg) return;
        const int i = pre.x;
        sfirst[i] = b;
        snb[i] = sg & 255;
        sdst[i] = on[b];
        sdoff[i] = jb[b];
        ssrc[i] = ja[b];
        srows[i] = sg >> 8;
        sunit[i] = pre.y;
        if (b == n_remote) misc[0] = i;   // the first local band starts a segment
      },
      sh);
  const int NS = stot.x, U = stot.y;
  const int n_rsegs = misc[0] >= 0 ? misc[0] : NS;
  if (tid == 0) sunit[NS] = U;

  // (g) gate/up m-tiles: the compacted rows of every X_e (its real rows,
  //     padding left out) cut into kGuBM-row tiles, experts in rule (ii)
  //     order; one thread per tile.  The GEMM computes no padding row.
  int32_t* mt_row = ws + L.o_gumt_row;
  int32_t* mt_exp = ws + L.o_gumt_exp;
  const int NMT = scan_items(
      E_l, [&](int q) { return (ce[order[q]] + kGuBM - 1) / kGuBM; },
      [&](int q, int pre) { gupre[q] = pre; }, sh);
  for (int t = tid; t < NMT; t += nt) {
    const int q = upper_index(gupre, E_l, t);
    const int e = order[q];
    mt_row[t] = crowoff[e] + (t - gupre[q]) * kGuBM;
    mt_exp[t] = e;
  }

  // (h) down tiles: the same 256-row pieces of every X_e's compacted rows
  //     as the gate/up tiles (X_e's remote groups first, then its local
  //     group), in schedule order: first every piece that holds remote rows,
  //     experts in rule (ii) order, then the pieces of local rows alone,
  //     experts ascending.  A piece may hold an expert's last remote rows and
  //     its first local rows, and a band may straddle two pieces: the GEMM's
  //     epilogue publishes the head and the tail of a band separately.  So
  //     the down GEMM runs as many row tiles as the gate/up GEMM, and none of
  //     them holds a padding row.
  int32_t* dt_row = ws + L.o_dnt_row;
  int32_t* dt_exp = ws + L.o_dnt_exp;
  int* dr = smem + S.dpre;    // [E_l]: pieces with remote rows before the q-th expert of rule (ii)
  int* dl = dr + E_l + 1;     // [E_l]: pieces of local rows alone before expert e
  auto rpieces = [&](int e) { return (ce[e] - c[e * W + r] + kDnBM - 1) / kDnBM; };
  const int NDR = scan_items(
      E_l, [&](int q) { return rpieces(order[q]); }, [&](int q, int pre) { dr[q] = pre; }, sh);
  const int NDT = NDR + scan_items(
      E_l, [&](int e) { return (ce[e] + kDnBM - 1) / kDnBM - rpieces(e); }, [&](int e, int pre) { dl[e] = pre; },
      sh);
  for (int t = tid; t < NDT; t += nt) {
    int e, j;
    if (t < NDR) {
      const int q = upper_index(dr, E_l, t);
      e = order[q];
      j = t - dr[q];
    } else {
      e = upper_index(dl, E_l, t - NDR);
      j = rpieces(e) + (t - NDR - dl[e]);
    }
    dt_row[t] = crowoff[e] + j * kDnBM;
    dt_exp[t] = e;
  }

  if (tid == 0) {
    hdr[H_M] = M;
    hdr[H_BANDS] = B;
    hdr[H_REMOTE] = n_remote;
    hdr[H_SEGS] = NS;
    hdr[H_RSEGS] = n_rsegs;
    hdr[H_GU_TILES] = NMT * L.gu_ntn;
    hdr[H_DN_TILES] = 2 * B * L.dn_tpb;
    hdr[H_UNITS] = U;
    hdr[H_RCOUNT] = rcount;
    hdr[H_GU_MT] = NMT;
    hdr[H_DN_MT] = NDT;
    hdr[H_DN_MT_R] = NDR;
  }
}

// In-wave stable rank of `v` among the lanes holding the same value
// (v in [0, 2^bits); lanes with v < 0 take no part): the lanes with equal
// values are found with one ballot per bit of v (a lane keeps the lanes that
// agree with it on every bit), so the cost is `bits` ballots whatever the
// number of distinct values.  The lowest lane of each value writes the wave's
// count of that value into cnt[v].
__device__ __forceinline__ int wave_match_rank(int v, int bits, int* cnt) {
  const int lane = threadIdx.x & 63;
  uint64_t same = __ballot(v >= 0);
  for (int i = 0; i < bits; ++i) {
    const bool bit = (v >> i) & 1;
    const uint64_t ones = __ballot(bit);
    same &= bit ? ones : ~ones;
  }
  if (v < 0) return 0;
  const int rank = __popcll(same & lanes_below(lane));
  if (rank == 0) cnt[v] = __popcll(same);
  return rank;
}

// bits needed for values in [0, n)
__device__ __forceinline__ int bits_for(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

// wait for the builder's tables: 2 s on the 100 MHz clock at most (the
// builder raises the word within microseconds; the bound only guarantees
// that every wave ends)
constexpr int64_t kPlanWaitTicks = 200000000;

// A pair placer (workgroups 1.. of the second launch): pair block b.  It
// first computes, from the histograms alone, its prefixes inside its owner
// (and, for the rank's own tokens, the owner-side slot bases); then it waits
// for the builder's group tables and gives every pair its stable rank inside
// its (expert, owner) group.
__device__ void place_pairs(const PlanLayout& L, const int32_t* __restrict__ topk, int32_t* __restrict__ ws,
                            int b) {
  extern __shared__ int smem[];
  const int tid = threadIdx.x, w = tid >> 6;
  constexpr int nt = kPlanThreads;
  const int o = owner_of_block(L, b);
  const int p0 = L.pair_off[o] + (b - L.blk_off[o]) * kPairsPerBlock;
  const int p1 = min(p0 + kPairsPerBlock, L.pair_off[o + 1]);
  const bool own = (o == L.r);
  const int E_l = L.E_l, E = L.E, W = L.W, HB = E_l + 2;
  const int NX = E_l + 1;              // local experts + "any local"
  const int nw = kPlanThreads / 64;
  const PlaceLds S = place_lds(E_l, E, nw);
  int* run = smem + S.run;             // [NX] running counts over the block's rounds
  int* wc = smem + S.wc;               // [nw][NX] per-wave counts of one round
  int* run_g = smem + S.run_g;         // [E] (own only)
  int* wc_g = smem + S.wc_g;           // [nw][E]
  int* bp = smem + S.bp;               // [E_l] pairs of the owner's earlier blocks per local expert
  int* pre_g = smem + S.pre_g;         // [E] own: pairs of the earlier own blocks per expert
  int* base_g = smem + S.base_g;       // [E] own: first slot of every expert's pairs
  int* srow = smem + S.srow;           // [E_l] first layout row of group (e, o)
  int* scrow = smem + S.scrow;         // [E_l] its first compacted row
  int* sh = smem + S.sh;
  int* misc = smem + S.misc;
  int32_t* hdr = ws + L.o_hdr;
  const int32_t* __restrict__ bh = ws + L.o_bh;
  const int32_t* __restrict__ bhr = ws + L.o_bhr;

  for (int i = tid; i < NX * (nw + 1); i += nt) smem[S.run + i] = 0;   // run and wc are adjacent
  if (own)
    for (int i = tid; i < E * (nw + 1); i += nt) smem[S.run_g + i] = 0;
  // (a) before the builder is ready: prefixes from the histograms
  int loc = 0;
  for (int e = tid; e < E_l; e += nt) {
    const int s = sum_blocks(bh, HB, e, L.blk_off[o], b);
    bp[e] = s;
    loc += s;
  }
  int before;   // local pairs in the owner's earlier blocks
  (void)block_scan(loc, sh, &before);
  if (own) {
    const int bo = b - L.blk_off[L.r];
    for (int g = tid; g < E; g += nt) {
      const int pre = sum_blocks(bhr, E, g, 0, bo);
      pre_g[g] = pre;
      base_g[g] = pre + sum_blocks(bhr, E, g, bo, L.NB_r);   // the own tokens' count of expert g
    }
    __syncthreads();
    (void)scan_items(
        E, [&](int g) { return base_g[g]; }, [&](int g, int pre) { base_g[g] = pre; }, sh);
  }
  // (b) wait for the builder
  if (tid == 0) {
    const uint64_t t0 = wall_clock64();
    int err = 0;
    while (agent_load(hdr + H_READY) == 0) {
      __builtin_amdgcn_s_sleep(2);
      if ((int64_t)(wall_clock64() - t0) > kPlanWaitTicks) { err = 4; break; }   // MOE_ETIMEOUT
    }
    if (err) agent_store(hdr + H_ERROR, err);
    else err = agent_load(hdr + H_ERROR);
    misc[0] = err;
  }
  __syncthreads();
  if (misc[0] != 0) return;
  // (c) the builder's tables for this owner's groups
  const int32_t* gc = ws + L.o_c;
  const int32_t* grow = ws + L.o_grow;
  const int32_t* gcrow = ws + L.o_gcrow;
  for (int e = tid; e < E_l; e += nt) {
    srow[e] = agent_load(grow + e * W + o);
    scrow[e] = agent_load(gcrow + e * W + o);
  }
  const int recv_base = agent_load(ws + L.o_obase + o) + before;
  int32_t* src = ws + L.o_src;
  // the padding entries of src_index: the tail of every remote group, the
  // groups shared out over the placers (groups b, b + NB, ...).  One thread
  // per group reads its size and first row (all of them in one round trip),
  // then the workgroup writes the -1 entries group by group
  {
    const int NGR = E_l * (W - 1);
    const int tb = L.tb_m;
    int* pst = smem + S.pst;
    int* pct = smem + S.pct;
    const int ng = NGR > b ? (NGR - b + L.NB - 1) / L.NB : 0;   // this placer's groups
    for (int j0 = 0; j0 < ng; j0 += nt) {
      const int j = j0 + tid;
      if (j < ng) {
        const int gi = b + j * L.NB;
        const int e = fdiv(gi, L.div_wm1), q = gi - e * (W - 1);
        const int og = q < L.r ? q : q + 1;
        const int n = agent_load(gc + e * W + og);
        pst[tid] = agent_load(grow + e * W + og) + n;
        pct[tid] = fdiv(n + tb - 1, L.div_tb) * tb - n;
      }
      __syncthreads();
      const int m = min(nt, ng - j0);
      for (int jj = 0; jj < m; ++jj) {
        const int st = pst[jj], ct = pct[jj];
        for (int x = tid; x < ct; x += nt) src[st + x] = -1;
      }
      __syncthreads();
    }
  }
  __syncthreads();   // srow, scrow complete
  int32_t* cmp_row = ws + L.o_cmprow;
  int32_t* cmp_src = ws + L.o_cmpsrc;
  int32_t* pos = ws + L.o_pos;
  const int lo = L.r * E_l;
  const int bits_e = bits_for(E_l + 1), bits_g = bits_for(E);
  for (int p_base = p0; p_base < p1; p_base += nt) {
    const int p = p_base + tid;
    const int g = (p < p1) ? topk[p] : -1;
    const int e = (g >= lo && g < lo + E_l) ? g - lo : -1;
    const int re = wave_match_rank(e, bits_e, wc + w * NX);
    const int rl = wave_match_rank(e >= 0 ? E_l : -1, bits_e, wc + w * NX);
    int rg = 0;
    if (own) rg = wave_match_rank((g >= 0 && g < E) ? g : -1, bits_g, wc_g + w * E);
    __syncthreads();
    if (e >= 0) {
      int rank_e = run[e] + re, rank_l = run[E_l] + rl;
      for (int x = 0; x < w; ++x) { rank_e += wc[x * NX + e]; rank_l += wc[x * NX + E_l]; }
      const int dest = srow[e] + bp[e] + rank_e;
      const int cdest = scrow[e] + bp[e] + rank_e;
      const int i = recv_base + rank_l;
      if (dest < L.rows_cap && i < L.R) src[dest] = i;
      if (cdest < L.R && i < L.R) {
        cmp_row[cdest] = dest;
        cmp_src[cdest] = i;
      }
    }
    if (own && g >= 0 && g < E) {
      int rank_g = run_g[g] + rg;
      for (int x = 0; x < w; ++x) rank_g += wc_g[x * E + g];
      pos[p - L.pair_off[L.r]] = base_g[g] + pre_g[g] + rank_g;
    }
    __syncthreads();
    for (int x = tid; x < NX; x += nt) {
      int s = 0;
      for (int y = 0; y < nw; ++y) { s += wc[y * NX + x]; wc[y * NX + x] = 0; }
      run[x] += s;
    }
    if (own)
      for (int x = tid; x < E; x += nt) {
        int s = 0;
        for (int y = 0; y < nw; ++y) { s += wc_g[y * E + x]; wc_g[y * E + x] = 0; }
        run_g[x] += s;
      }
    __syncthreads();
  }
}

// The second launch: workgroup 0 builds the plan, workgroups 1..NB place
// the pairs of one block each.  The builder has the lowest id, so it is
// dispatched first and never waits for a placer.
__global__ __launch_bounds__(kPlanThreads) void plan_build_place_kernel(PlanLayout L, const int32_t* __restrict__ topk,
                                                                       int32_t* __restrict__ ws) {
  if (blockIdx.x == 0) {
    if (L.band_lds) build_plan<true>(L, ws);
    else build_plan<false>(L, ws);
  } else {
    place_pairs(L, topk, ws, blockIdx.x - 1);
  }
}

// Raw buffer resource over [base, base + bytes): loads past the end read
// zero, stores past it are dropped (gfx9-family word 3: 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef unsigned int gv4u32 __attribute__((ext_vector_type(4)));

#ifndef MOE_GATHER_STORE_AUX
#define MOE_GATHER_STORE_AUX 0   // cache-policy bits of the layout stores
#endif

// One wavefront per layout row: a real row is copied from x_recv with
// kGatherBatch 16-byte loads per lane in flight before their stores; a
// padding row is written as zeros.  Both ends are bounded by per-row buffer
// descriptors, so a row length that is not a multiple of the batch needs
// no branch.
constexpr int kGatherBatch = 8;

__global__ __launch_bounds__(256) void plan_gather_kernel(PlanLayout L, const int32_t* __restrict__ ws,
                                                         const uint16_t* __restrict__ x_recv,
                                                         uint16_t* __restrict__ x_layout) {
  const int32_t* hdr = ws + L.o_hdr;
  if (hdr[H_ERROR] != 0) return;
  const int M = hdr[H_M];
  const int32_t* src = ws + L.o_src;
  const int lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;
  const int64_t row_bytes = (int64_t)L.d * 2;
  for (int row = blockIdx.x * wpb + (threadIdx.x >> 6); row < M; row += gridDim.x * wpb) {
    const int s = src[row];
    const __amdgpu_buffer_rsrc_t dst = row_rsrc(x_layout + (int64_t)row * L.d, row_bytes);
    if (s >= 0) {
      const __amdgpu_buffer_rsrc_t sp = row_rsrc(x_recv + (int64_t)s * L.d, row_bytes);
      for (int b0 = 0; b0 < row_bytes; b0 += kGatherBatch * 64 * 16) {
        gv4u32 v[kGatherBatch];
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u)
          v[u] = __builtin_amdgcn_raw_buffer_load_b128(sp, b0 + (u * 64 + lane) * 16, 0, 0);
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(v[u], dst, b0 + (u * 64 + lane) * 16, 0, MOE_GATHER_STORE_AUX);
      }
    } else {
      const gv4u32 z = {0u, 0u, 0u, 0u};
      for (int b0 = 0; b0 < row_bytes; b0 += kGatherBatch * 64 * 16) {
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(z, dst, b0 + (u * 64 + lane) * 16, 0, MOE_GATHER_STORE_AUX);
      }
    }
  }
}

}  // namespace

hipError_t launch_plan(const PlanLayout& L, const int32_t* topk, const uint16_t* x_recv, int32_t* ws,
                       uint16_t* x_layout, hipStream_t s) {
  if (L.NB > 0) {
    const size_t sh_count = (size_t)(L.E_l + 2 + L.E) * sizeof(int);
    hipLaunchKernelGGL(plan_count_kernel, dim3(L.NB), dim3(kPlanThreads), sh_count, s, L, topk, ws);
  }
  const int words = max(build_lds(L.W, L.E_l, L.bands_cap, L.band_lds != 0).total,
                        L.NB > 0 ? place_lds(L.E_l, L.E, kPlanThreads / 64).total : 0);
  hipLaunchKernelGGL(plan_build_place_kernel, dim3(1 + L.NB), dim3(kPlanThreads), (size_t)words * sizeof(int), s, L,
                     topk, ws);
  if (x_layout == nullptr) return hipGetLastError();   // metadata only: the GEMM gathers its rows
  const int rows_per_block = 4;
  int grid = (L.rows_cap + rows_per_block - 1) / rows_per_block;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(plan_gather_kernel, dim3(grid), dim3(256), 0, s, L, (const int32_t*)ws, x_recv, x_layout);
  return hipGetLastError();
}

}  // namespace moe
