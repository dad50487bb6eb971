// Planner: Stage A of the tile-signal notes ("MoE 计算-通信细粒度重叠：用 Tile 级信号把
// All-to-All 藏在 GEMM 背后", §3 and §4.2-§4.5, segments §5.2), on the device.
//
//   K1 plan_count   one workgroup per 512 (token, slot) pairs of one owner:
//                   LDS histograms of the local experts, of "below this rank's
//                   experts" (for receive offsets) and, for the rank's own
//                   tokens, of all experts (for the owner-side slot table).
//   K2 plan_build   one workgroup of 256 threads: scans over the histograms
//                   -> group counts, padded group offsets, X_e sizes, rule
//                   (ii) expert order, band list S (remote bands first),
//                   combine plan, segments and their copy units, GEMM row-tile
//                   tables, padding extent of every remote group.  Its tables
//                   live in LDS; nothing it writes to memory is read back.
//   K3 plan_place   one workgroup per pair block again: stable rank of every
//                   pair inside its (expert, owner) group with bit-sliced wave
//                   ballots + LDS carries -> src_index of every real layout
//                   row, and the owner-side slot of each of the rank's own
//                   pairs; the blocks also write the padding entries (-1).
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

// Exclusive scan of a pair of ints per thread over the workgroup (at most
// kBuildThreads threads): wavefront scans, then every thread adds the totals
// of the wavefronts below its own (read in parallel from LDS).  `sh` holds
// 2 ints per wavefront.  Two barriers; `sh` is free again on return.
__device__ int2 block_scan2(int a, int b, int* sh, int2* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = (blockDim.x + 63) >> 6;
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
  const int per = (n + blockDim.x - 1) / blockDim.x;
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
  const int per = (n + blockDim.x - 1) / blockDim.x;
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

__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(PlanLayout L, const int32_t* __restrict__ topk,
                                                                 int32_t* __restrict__ ws) {
  extern __shared__ int sh[];
  const int b = blockIdx.x;
  const int o = owner_of_block(L, b);
  const int p0 = L.pair_off[o] + (b - L.blk_off[o]) * kPairsPerBlock;
  const int p1 = min(p0 + kPairsPerBlock, L.pair_off[o + 1]);
  const bool own = (o == L.r);
  const int nb = L.E_l + 2 + (own ? L.E : 0);
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

__global__ __launch_bounds__(kBuildThreads) void plan_build_kernel(PlanLayout L, int32_t* __restrict__ ws) {
  extern __shared__ int smem[];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int W = L.W, r = L.r, E_l = L.E_l, E = L.E, tb = L.tb_m;
  const int HB = E_l + 2;
  const int EW = E_l * W;
  const BuildLds S = build_lds(W, E_l, E, L.NB, L.NB_r, L.band_table, L.build_stage != 0);
  int32_t* hdr = ws + L.o_hdr;
  int* c = smem + S.c;             // [E_l][W] group sizes
  int* grp = smem + S.grp;         // [E_l][W] group offsets inside X_e
  int* base = smem + S.base;       // [W][E_l] receive-buffer bases
  int* gstart = smem + S.gstart;   // [E_l*W + 1] first band of every group in S order
  int* low = smem + S.low;         // [W]
  int* me = smem + S.me;           // [E_l]
  int* rowoff = smem + S.rowoff;   // [E_l + 1]
  int* rb = smem + S.rb;           // [E_l]
  int* order = smem + S.order;     // [E_l]
  int* baser = smem + S.baser;     // [E]
  int* gupre = smem + S.gupre;     // [E_l + 1] gate/up row tiles before each expert (rule (ii) order)
  int* dnpre = smem + S.dnpre;     // [2 E_l + 1] down row tiles before each run
  int* sh = smem + S.sh;           // scan scratch
  int* misc = smem + S.misc;       // [0] remote segments
  int* ccum = smem + S.ccum;       // [E_l][W] group offsets inside X_e's compacted rows
  int* ce = smem + S.ce;           // [E_l] real rows of X_e
  int* crowoff = smem + S.crowoff; // [E_l + 1] first compacted row of X_e
  const int32_t* bh = ws + L.o_bh;
  int32_t* bp = ws + L.o_bp;
  int32_t* brecv = ws + L.o_brecv;
  const int32_t* bhr = ws + L.o_bhr;
  int32_t* bpr = ws + L.o_bpr;
  if (L.build_stage) {
    // the per-block histograms are read many times below: one coalesced
    // parallel copy into LDS (the host sized the LDS for it)
    int* s_bh = smem + S.stage_bh;
    int* s_bhr = smem + S.stage_bhr;
    // 16-byte loads, 8 in flight per thread (both ends 16-byte aligned);
    // the last n mod 4 words one by one
    auto stage = [&](int* dst, const int32_t* src, int n) {
      const int n4 = n >> 2;
      const int4* s4 = (const int4*)src;
      int4* d4 = (int4*)dst;
      for (int i0 = tid; i0 < n4; i0 += 8 * nt) {
        int4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u * nt < n4) v[u] = s4[i0 + u * nt];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u * nt < n4) d4[i0 + u * nt] = v[u];
      }
      for (int i = 4 * n4 + tid; i < n; i += nt) dst[i] = src[i];
    };
    stage(s_bh, bh, L.NB * HB);
    stage(s_bhr, bhr, L.NB_r * E);
    __syncthreads();
    bh = s_bh;
    bhr = s_bhr;
  }

  // (a) received-row base of every block (owners in order) and routing
  //     errors, in one scan over the blocks
  const int2 rtot = scan_items2(
      L.NB,
      [&](int b) {
        int s = 0;
        for (int e = 0; e < E_l; ++e) s += bh[(int64_t)b * HB + e];
        return make_int2(s, bh[(int64_t)b * HB + E_l + 1]);
      },
      [&](int b, int2 pre) { brecv[b] = pre.x; }, sh);
  const int rcount = rtot.x, bad_total = rtot.y;

  // (b) group counts c[e][o], low[o], per-block prefixes within each owner
  // (the histogram entries are loaded 8 at a time ahead of the dependent
  // stores, which the compiler cannot move past loads from the same workspace)
  for (int it = tid; it < W * (E_l + 1); it += nt) {
    const int o = it / (E_l + 1), x = it % (E_l + 1);
    int run = 0;
    for (int b0 = L.blk_off[o]; b0 < L.blk_off[o + 1]; b0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (b0 + u < L.blk_off[o + 1]) ? bh[(int64_t)(b0 + u) * HB + x] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < L.blk_off[o + 1]) bp[(int64_t)(b0 + u) * (E_l + 1) + x] = run;
        run += v[u];
      }
    }
    if (x < E_l) c[x * W + o] = run; else low[o] = run;
  }
  // (c) the rank's own tokens: per-expert counts and per-block prefixes
  for (int g = tid; g < E; g += nt) {
    int run = 0;
    for (int b0 = 0; b0 < L.NB_r; b0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (b0 + u < L.NB_r) ? bhr[(int64_t)(b0 + u) * E + g] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < L.NB_r) bpr[(int64_t)(b0 + u) * E + g] = run;
        run += v[u];
      }
    }
    baser[g] = run;  // count for now, turned into a prefix below
  }
  __syncthreads();
  (void)scan_items(
      E, [&](int g) { return baser[g]; }, [&](int g, int pre) { baser[g] = pre; }, sh);

  if (bad_total > 0 || rcount != L.R) {
    if (tid == 0) {
      hdr[H_ERROR] = 5;  // MOE_EROUTING
      for (int i = 1; i < H_WORDS; ++i) hdr[i] = 0;
      hdr[H_RCOUNT] = rcount;
    }
    return;
  }

  // (d) layout: padded group offsets inside X_e, remote owners ascending then
  //     r; receive-buffer bases: owner o's pairs below global expert r*E_l + e
  for (int e = tid; e < E_l; e += nt) {
    int run = 0, crun = 0;
    for (int q = 0; q < W; ++q) {
      const int o = (q < W - 1) ? (q < r ? q : q + 1) : r;
      grp[e * W + o] = run;
      ccum[e * W + o] = crun;
      const int n = c[e * W + o];
      run += (o == r) ? n : ((n + tb - 1) / tb) * tb;
      crun += n;
    }
    me[e] = run;
    ce[e] = crun;
  }
  for (int o = tid; o < W; o += nt) {
    int run = low[o];
    for (int e = 0; e < E_l; ++e) { base[o * E_l + e] = run; run += c[e * W + o]; }
  }
  // remote bands per expert, for rule (ii)
  for (int e = tid; e < E_l; e += nt) {
    int n = 0;
    for (int o = 0; o < W; ++o)
      if (o != r) n += (c[e * W + o] + tb - 1) / tb;
    rb[e] = n;
  }
  __syncthreads();
  const int2 mtot = scan_items2(
      E_l, [&](int e) { return make_int2(me[e], ce[e]); },
      [&](int e, int2 pre) {
        rowoff[e] = pre.x;
        crowoff[e] = pre.y;
      },
      sh);
  const int M = mtot.x;
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
  if (tid == 0) {
    rowoff[E_l] = M;
    crowoff[E_l] = mtot.y;   // = rcount
  }
  __syncthreads();

  // (e) groups in schedule order: remote groups of experts in rule (ii) order
  //     (owners ascending, r skipped), then the local group of every expert.
  const int NGR = E_l * (W - 1);
  const int NG = E_l * W;
  auto group_eo = [&](int gi, int& e, int& o) {
    if (gi < NGR) {
      e = order[gi / (W - 1)];
      const int q = gi % (W - 1);
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
        return (c[e * W + o] + tb - 1) / tb;
      },
      [&](int gi, int pre) { gstart[gi] = pre; }, sh);
  if (B > L.bands_cap) {
    if (tid == 0) { hdr[H_ERROR] = 2; for (int i = 1; i < H_WORDS; ++i) hdr[i] = 0; }
    return;
  }
  const int n_remote = NGR < NG ? gstart[NGR] : B;

  // (f) bands in S order, one thread per group (a group's bands are
  //     consecutive in S), a band -> group table in LDS when it fits, and
  //     the padding rows of every remote group
  int32_t* bexp = ws + L.o_bexp;
  int32_t* bdst = ws + L.o_bdst;
  int32_t* bsrc = ws + L.o_bsrc;
  int32_t* bdoff = ws + L.o_bdoff;
  int32_t* bval = ws + L.o_bval;
  int32_t* bcrow = ws + L.o_bcrow;
  int* band_g = L.band_table > 0 ? smem + S.band_g : nullptr;
  int32_t* pad_st = ws + L.o_pad;         // read by plan_place, which writes the padding entries
  int32_t* pad_ct = pad_st + EW;
  for (int gi = tid; gi < NG; gi += nt) {
    int e, o;
    group_eo(gi, e, o);
    const int n = c[e * W + o];
    const int nb = (n + tb - 1) / tb;
    const int gs = gstart[gi];
    const int rowb = rowoff[e] + grp[e * W + o];
    const int dstb = base[o * E_l + e];
    const int crowb = crowoff[e] + ccum[e * W + o];
    for (int q = 0; q < nb; ++q) {
      if (band_g) band_g[gs + q] = gi;
      bcrow[gs + q] = crowb + q * tb;
      bexp[gs + q] = e;
      bdst[gs + q] = o;
      bsrc[gs + q] = rowb + q * tb;
      bdoff[gs + q] = dstb + q * tb;
      bval[gs + q] = min(tb, n - q * tb);
    }
    if (gi < NGR) {
      pad_st[gi] = rowb + n;
      pad_ct[gi] = nb * tb - n;
    }
  }

  // (g) segments (§5.2): the first and the last remote band alone; otherwise
  //     runs of <= mgb bands that restart at every group boundary.  Every
  //     band decides whether it starts a segment and, if so, the segment's
  //     bands, rows and copy units (a segment never crosses a group, so they
  //     are read off the group); one pair scan over the bands numbers the
  //     segments and places their copy units.
  const int mgb = L.mgb;
  const int64_t row_bytes = (int64_t)L.d * 2;
  auto units_of = [&](int rows) { return (int)((rows * row_bytes + kCopyChunk - 1) / kCopyChunk); };
  if (tid == 0) gstart[NG] = B;
  __syncthreads();   // band table, gstart[NG]
  auto group_of = [&](int b) { return band_g ? band_g[b] : upper_index(gstart, NG, b); };
  // does band b (of group gi, first band gs) start a segment
  auto starts = [&](int b, int gi, int gs) {
    if (b == gs) return true;
    if (gi < NGR) {
      const int run0 = gs > 1 ? gs : 1;
      return b == n_remote - 1 || ((b - run0) % mgb) == 0;
    }
    return ((b - gs) % mgb) == 0;
  };
  // segment starting at band b: its bands and rows (false if b starts none)
  auto seg_at = [&](int b, int& gi, int& nb, int& rows) {
    gi = group_of(b);
    const int gs = gstart[gi];
    if (!starts(b, gi, gs)) return false;
    const int ge = gstart[gi + 1];
    nb = 1;
    while (b + nb < ge && !starts(b + nb, gi, gs)) ++nb;
    int e, o;
    group_eo(gi, e, o);
    rows = min(nb * tb, c[e * W + o] - (b - gs) * tb);
    return true;
  };
  int32_t* sfirst = ws + L.o_sfirst;
  int32_t* snb = ws + L.o_snb;
  int32_t* sdst = ws + L.o_sdst;
  int32_t* sdoff = ws + L.o_sdoff;
  int32_t* ssrc = ws + L.o_ssrc;
  int32_t* srows = ws + L.o_srows;
  int32_t* sunit = ws + L.o_sunit;
  if (tid == 0) misc[0] = -1;
  __syncthreads();
  const int2 stot = scan_items2(
      B,
      [&](int b) {
        int gi, nb, rows;
        if (!seg_at(b, gi, nb, rows)) return make_int2(0, 0);
        return make_int2(1, units_of(rows));
      },
      [&](int b, int2 pre) {
        int gi, nb, rows;
        if (!seg_at(b, gi, nb, rows)) return;
        int e, o;
        group_eo(gi, e, o);
        const int q = b - gstart[gi];
        const int i = pre.x;
        sfirst[i] = b;
        snb[i] = nb;
        sdst[i] = o;
        sdoff[i] = base[o * E_l + e] + q * tb;
        ssrc[i] = rowoff[e] + grp[e * W + o] + q * tb;
        srows[i] = rows;
        sunit[i] = pre.y;
        if (b == n_remote) misc[0] = i;   // the first local band starts a segment
      },
      sh);
  const int NS = stot.x, U = stot.y;
  const int n_rsegs = misc[0] >= 0 ? misc[0] : NS;
  if (tid == 0) sunit[NS] = U;

  // (i) gate/up m-tiles: the compacted rows of every X_e (its real rows,
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

  // (j) down tiles: the runs of row-contiguous bands in S order -- the
  //     remote bands of each expert in rule (ii) order (its remote groups
  //     follow one another at the start of X_e), then the local bands of
  //     each expert -- each cut greedily into tiles of whole bands whose
  //     real rows add up to at most kDnBM (and at most kDnMaxBands bands).
  //     The GEMM multiplies a tile's real rows only, packed, so a tile of
  //     two half-empty bands costs one band's work.  One thread per run:
  //     count, scan, then write.
  int32_t* dt_row = ws + L.o_dnt_row;
  int32_t* dt_exp = ws + L.o_dnt_exp;
  int32_t* dt_band = ws + L.o_dnt_band;
  int32_t* dt_nb = ws + L.o_dnt_nb;
  // greedy packing of run q; with `at` >= 0 the tiles are written from
  // index `at` on; returns the number of tiles
  auto pack_run = [&](int q, int at) {
    const bool remote_run = q < E_l;
    const int e = remote_run ? order[q] : q - E_l;
    int b = remote_run ? (W > 1 ? gstart[q * (W - 1)] : 0) : gstart[NGR + e];
    int ntiles = 0, rows = 0, nbt = 0, tfirst = b, trow = 0;
    for (int qq = 0; qq < W; ++qq) {
      int o;
      if (remote_run) {
        if (qq >= W - 1) break;
        o = qq < r ? qq : qq + 1;
      } else {
        if (qq > 0) break;
        o = r;
      }
      const int n = c[e * W + o];
      const int row_g = rowoff[e] + grp[e * W + o];
      for (int j = 0; j * tb < n; ++j, ++b) {
        const int v = min(tb, n - j * tb);
        if (nbt > 0 && (rows + v > kDnBM || nbt == kDnMaxBands)) {
          if (at >= 0) {
            dt_row[at + ntiles] = trow;
            dt_exp[at + ntiles] = e;
            dt_band[at + ntiles] = tfirst;
            dt_nb[at + ntiles] = nbt;
          }
          ++ntiles;
          rows = 0;
          nbt = 0;
        }
        if (nbt == 0) {
          tfirst = b;
          trow = row_g + j * tb;
        }
        rows += v;
        ++nbt;
      }
    }
    if (nbt > 0) {
      if (at >= 0) {
        dt_row[at + ntiles] = trow;
        dt_exp[at + ntiles] = e;
        dt_band[at + ntiles] = tfirst;
        dt_nb[at + ntiles] = nbt;
      }
      ++ntiles;
    }
    return ntiles;
  };
  const int NDT = scan_items(
      2 * E_l, [&](int q) { return pack_run(q, -1); }, [&](int q, int pre) { dnpre[q] = pre; }, sh);
  const int ndt_r = dnpre[E_l];   // the remote runs come first
  for (int q = tid; q < 2 * E_l; q += nt) (void)pack_run(q, dnpre[q]);

  // results used by later kernels and by inspection
  for (int i = tid; i < EW; i += nt) {
    ws[L.o_c + i] = c[i];
    ws[L.o_grp + i] = grp[i];
    ws[L.o_base + i] = base[i];
    ws[L.o_ccum + i] = ccum[i];
  }
  for (int i = tid; i <= E_l; i += nt) ws[L.o_crowoff + i] = crowoff[i];
  for (int i = tid; i < W; i += nt) ws[L.o_low + i] = low[i];
  for (int i = tid; i < E_l; i += nt) {
    ws[L.o_me + i] = me[i];
    ws[L.o_rb + i] = rb[i];
    ws[L.o_order + i] = order[i];
  }
  for (int i = tid; i <= E_l; i += nt) ws[L.o_rowoff + i] = rowoff[i];
  for (int i = tid; i < E; i += nt) ws[L.o_baser + i] = baser[i];
  if (tid == 0) {
    hdr[H_ERROR] = 0;
    hdr[H_M] = M;
    hdr[H_BANDS] = B;
    hdr[H_REMOTE] = n_remote;
    hdr[H_SEGS] = NS;
    hdr[H_RSEGS] = n_rsegs;
    hdr[H_GU_TILES] = NMT * L.gu_ntn;
    hdr[H_DN_TILES] = B * L.dn_tpb;
    hdr[H_UNITS] = U;
    hdr[H_RCOUNT] = rcount;
    hdr[H_GU_MT] = NMT;
    hdr[H_DN_MT] = NDT;
    hdr[H_DN_MT_R] = ndt_r;
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

__global__ __launch_bounds__(kPlanThreads) void plan_place_kernel(PlanLayout L, const int32_t* __restrict__ topk,
                                                                 int32_t* __restrict__ ws) {
  extern __shared__ int sh[];
  const int32_t* hdr = ws + L.o_hdr;
  if (hdr[H_ERROR] != 0) return;
  const int b = blockIdx.x;
  const int o = owner_of_block(L, b);
  const int p0 = L.pair_off[o] + (b - L.blk_off[o]) * kPairsPerBlock;
  const int p1 = min(p0 + kPairsPerBlock, L.pair_off[o + 1]);
  const bool own = (o == L.r);
  const int E_l = L.E_l, E = L.E, W = L.W;
  const int NX = E_l + 1;              // local experts + "any local"
  const int nw = kPlanThreads / 64;
  int* run = sh;                       // [NX]
  int* wc = run + NX;                  // [nw][NX]
  int* run_g = wc + nw * NX;           // [E] (own only)
  int* wc_g = run_g + E;               // [nw][E]
  const int tid = threadIdx.x, w = tid >> 6;
  for (int i = tid; i < NX * (nw + 1); i += blockDim.x) sh[i] = 0;
  if (own)
    for (int i = tid; i < E * (nw + 1); i += blockDim.x) run_g[i] = 0;
  __syncthreads();
  const int32_t* rowoff = ws + L.o_rowoff;
  const int32_t* grp = ws + L.o_grp;
  const int32_t* crowoff = ws + L.o_crowoff;
  const int32_t* ccum = ws + L.o_ccum;
  int32_t* cmp_row = ws + L.o_cmprow;
  int32_t* cmp_src = ws + L.o_cmpsrc;
  const int32_t* bp = ws + L.o_bp + (int64_t)b * (E_l + 1);
  const int recv_base = ws[L.o_brecv + b];
  int32_t* src = ws + L.o_src;
  const int32_t* bpr = ws + L.o_bpr + (int64_t)(b - L.blk_off[L.r]) * E;
  const int32_t* baser = ws + L.o_baser;
  int32_t* pos = ws + L.o_pos;
  // the padding entries of src_index: the tail of every remote group, the
  // groups shared out over the blocks
  {
    const int NGR = E_l * (W - 1);
    const int32_t* pad_st = ws + L.o_pad;
    const int32_t* pad_ct = pad_st + E_l * W;
    for (int gi = blockIdx.x; gi < NGR; gi += gridDim.x) {
      const int st = pad_st[gi], ct = pad_ct[gi];
      for (int q = threadIdx.x; q < ct; q += blockDim.x) src[st + q] = -1;
    }
  }
  const int lo = L.r * E_l;
  const int bits_e = bits_for(E_l + 1), bits_g = bits_for(E);
  for (int p_base = p0; p_base < p1; p_base += blockDim.x) {
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
      const int dest = rowoff[e] + grp[e * W + o] + bp[e] + rank_e;
      const int cdest = crowoff[e] + ccum[e * W + o] + bp[e] + rank_e;
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
      pos[p - L.pair_off[L.r]] = baser[g] + bpr[g] + rank_g;
    }
    __syncthreads();
    for (int x = tid; x < NX; x += blockDim.x) {
      int s = 0;
      for (int y = 0; y < nw; ++y) { s += wc[y * NX + x]; wc[y * NX + x] = 0; }
      run[x] += s;
    }
    if (own)
      for (int x = tid; x < E; x += blockDim.x) {
        int s = 0;
        for (int y = 0; y < nw; ++y) { s += wc_g[y * E + x]; wc_g[y * E + x] = 0; }
        run_g[x] += s;
      }
    __syncthreads();
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
  const int words = build_lds(L.W, L.E_l, L.E, L.NB, L.NB_r, L.band_table, L.build_stage != 0).total;
  hipLaunchKernelGGL(plan_build_kernel, dim3(1), dim3(kBuildThreads), (size_t)words * sizeof(int), s, L, ws);
  if (L.NB > 0) {
    const int nw = kPlanThreads / 64;
    const size_t sh_place = (size_t)((L.E_l + 1) * (nw + 1) + L.E * (nw + 1)) * sizeof(int);
    hipLaunchKernelGGL(plan_place_kernel, dim3(L.NB), dim3(kPlanThreads), sh_place, s, L, topk, ws);
  }
  if (x_layout == nullptr) return hipGetLastError();   // metadata only: the GEMM gathers its rows
  const int rows_per_block = 4;
  int grid = (L.rows_cap + rows_per_block - 1) / rows_per_block;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(plan_gather_kernel, dim3(grid), dim3(256), 0, s, L, (const int32_t*)ws, x_recv, x_layout);
  return hipGetLastError();
}

}  // namespace moe
