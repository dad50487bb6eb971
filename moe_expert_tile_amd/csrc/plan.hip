// Planner: Stage A of the tile-signal notes ("MoE 计算-通信细粒度重叠：用 Tile 级信号把
// All-to-All 藏在 GEMM 背后", §3 and §4.2-§4.5, segments §5.2), on the device.
//
//   K1 plan_count   one workgroup per 2048 (token, slot) pairs of one owner:
//                   LDS histograms of the local experts, of "below this rank's
//                   experts" (for receive offsets) and, for the rank's own
//                   tokens, of all experts (for the owner-side slot table).
//   K2 plan_build   one workgroup: scans over the histograms -> group counts,
//                   padded group offsets, X_e sizes, rule (ii) expert order,
//                   band list S (remote bands first), combine plan, segments,
//                   gate/up tile table, padding entries of src_index.
//   K3 plan_place   one workgroup per pair block again: stable rank of every
//                   pair inside its (expert, owner) group with wave ballots +
//                   LDS carries -> src_index of every real layout row, and the
//                   owner-side slot of each of the rank's own pairs.
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

// Exclusive scan of one int per thread over the whole workgroup.
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < nw; ++i) { int t = sh[i]; sh[i] = run; run += t; }
    sh[32] = run;
  }
  __syncthreads();
  int res = sh[w] + x - v;
  *total = sh[32];
  __syncthreads();
  return res;
}

// Exclusive scan over n items: val(i) gives item i, out(i, prefix) receives
// its exclusive prefix.  Items are split into contiguous per-thread chunks.
template <class F, class G>
__device__ int scan_items(int n, F val, G out, int* sh) {
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += val(i);
  int total;
  int run = block_excl_scan(local, sh, &total);
  for (int i = lo; i < hi; ++i) { int v = val(i); out(i, run); run += v; }
  __syncthreads();
  return total;
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
  int32_t* hdr = ws + L.o_hdr;
  int* c = smem;                 // [E_l][W]
  int* grp = c + EW;             // [E_l][W]
  int* base = grp + EW;          // [W][E_l]
  int* gstart = base + EW;       // [E_l*W] per-group band start
  int* gseg = gstart + EW;       // [E_l*W] per-group segment base
  int* gunit = gseg + EW;        // [E_l*W] per-group copy-unit base
  int* low = gunit + EW;         // [W]
  int* me = low + W;             // [E_l]
  int* rowoff = me + E_l;        // [E_l + 1]
  int* rb = rowoff + E_l + 1;    // [E_l]
  int* order = rb + E_l;         // [E_l]
  int* baser = order + E_l;      // [E]
  int* sh = baser + E;           // [64] scan scratch
  const int32_t* bh = ws + L.o_bh;
  int32_t* bp = ws + L.o_bp;
  int32_t* brecv = ws + L.o_brecv;
  const int32_t* bhr = ws + L.o_bhr;
  int32_t* bpr = ws + L.o_bpr;
  if (L.build_stage) {
    // the per-block histograms are read many times below: one coalesced
    // parallel copy into LDS, after the tables (the host sized the LDS for it)
    int* s_bh = sh + 64;
    int* s_bhr = s_bh + L.NB * HB;
    for (int i = tid; i < L.NB * HB; i += nt) s_bh[i] = bh[i];
    for (int i = tid; i < L.NB_r * E; i += nt) s_bhr[i] = bhr[i];
    __syncthreads();
    bh = s_bh;
    bhr = s_bhr;
  }

  // (a) routing errors
  int bad_local = 0;
  for (int b = tid; b < L.NB; b += nt) bad_local += bh[(int64_t)b * HB + E_l + 1];
  int bad_total;
  (void)block_excl_scan(bad_local, sh, &bad_total);

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
  // (c) received-row base of every block
  int rcount = scan_items(
      L.NB,
      [&](int b) {
        int s = 0;
        for (int e = 0; e < E_l; ++e) s += bh[(int64_t)b * HB + e];
        return s;
      },
      [&](int b, int pre) { brecv[b] = pre; }, sh);
  // (d) the rank's own tokens: per-expert counts and per-block prefixes
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
  // scan_items reads item g (val) before it calls out(g), so the counts can be
  // replaced by their prefixes in place

  if (bad_total > 0 || rcount != L.R) {
    if (tid == 0) {
      hdr[H_ERROR] = 5;  // MOE_EROUTING
      for (int i = 1; i < H_WORDS; ++i) hdr[i] = 0;
      hdr[H_RCOUNT] = rcount;
    }
    return;
  }

  // (e) layout: padded group offsets inside X_e, remote owners ascending then r
  for (int e = tid; e < E_l; e += nt) {
    int run = 0;
    for (int q = 0; q < W; ++q) {
      const int o = (q < W - 1) ? (q < r ? q : q + 1) : r;
      grp[e * W + o] = run;
      const int n = c[e * W + o];
      run += (o == r) ? n : ((n + tb - 1) / tb) * tb;
    }
    me[e] = run;
  }
  // receive-buffer bases: owner o's pairs below global expert r*E_l + e
  for (int o = tid; o < W; o += nt) {
    int run = low[o];
    for (int e = 0; e < E_l; ++e) { base[o * E_l + e] = run; run += c[e * W + o]; }
  }
  __syncthreads();
  const int M = scan_items(
      E_l, [&](int e) { return me[e]; }, [&](int e, int pre) { rowoff[e] = pre; }, sh);
  if (tid == 0) rowoff[E_l] = M;
  // remote bands per expert and rule (ii) order: more remote bands first, ties to lower id
  for (int e = tid; e < E_l; e += nt) {
    int n = 0;
    for (int o = 0; o < W; ++o)
      if (o != r) n += (c[e * W + o] + tb - 1) / tb;
    rb[e] = n;
  }
  __syncthreads();
  for (int e = tid; e < E_l; e += nt) {
    int rank = 0;
    const int mine = rb[e];
    for (int x = 0; x < E_l; ++x) {
      const int v = rb[x];
      rank += (v > mine) || (v == mine && x < e);
    }
    order[rank] = e;
  }
  __syncthreads();

  // (f) groups in schedule order: remote groups of experts in rule (ii) order
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
  auto group_nb = [&](int gi) {
    int e, o;
    group_eo(gi, e, o);
    return (c[e * W + o] + tb - 1) / tb;
  };
  const int B = scan_items(NG, group_nb, [&](int gi, int pre) { gstart[gi] = pre; }, sh);
  int nrem_local = 0;
  for (int gi = tid; gi < NGR; gi += nt) nrem_local += group_nb(gi);
  int n_remote;
  (void)block_excl_scan(nrem_local, sh, &n_remote);
  if (B > L.bands_cap) {
    if (tid == 0) { hdr[H_ERROR] = 2; for (int i = 1; i < H_WORDS; ++i) hdr[i] = 0; }
    return;
  }

  // (g) bands in S order, one thread per band.  Band s belongs to the last
  //     group whose first band is <= s (that group is never empty).
  int32_t* bexp = ws + L.o_bexp;
  int32_t* bdst = ws + L.o_bdst;
  int32_t* bsrc = ws + L.o_bsrc;
  int32_t* bdoff = ws + L.o_bdoff;
  int32_t* bval = ws + L.o_bval;
  auto group_of = [&](int band) {
    int lo = 0, hi = NG - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gstart[mid] <= band) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  for (int b = tid; b < B; b += nt) {
    const int gi = group_of(b);
    int e, o;
    group_eo(gi, e, o);
    const int q = b - gstart[gi];
    bexp[b] = e;
    bdst[b] = o;
    bsrc[b] = rowoff[e] + grp[e * W + o] + q * tb;
    bdoff[b] = base[o * E_l + e] + q * tb;
    bval[b] = min(tb, c[e * W + o] - q * tb);
  }
  __syncthreads();   // the band arrays are read back below

  // segments (§5.2): the first and the last remote band alone; otherwise runs
  // of <= mgb bands that restart at every group boundary.  Every band decides
  // whether it starts a segment; a scan numbers the starts; each segment then
  // reads its fields off its first band (segments never cross a group, so the
  // first band's destination offset and source row are the segment's) and
  // sums its <= 64 bands' valid rows; a second scan places the copy units.
  const int mgb = L.mgb;
  auto starts_segment = [&](int b) {
    const int gi = group_of(b);
    const int gs = gstart[gi];
    if (b == gs) return 1;
    if (gi < NGR) {
      if (b == n_remote - 1) return 1;
      const int run0 = gs > 1 ? gs : 1;
      return ((b - run0) % mgb) == 0 ? 1 : 0;
    }
    return ((b - gs) % mgb) == 0 ? 1 : 0;
  };
  const int64_t row_bytes = (int64_t)L.d * 2;
  auto units_of = [&](int rows) { return (int)((rows * row_bytes + kCopyChunk - 1) / kCopyChunk); };
  int32_t* sfirst = ws + L.o_sfirst;
  int32_t* snb = ws + L.o_snb;
  int32_t* sdst = ws + L.o_sdst;
  int32_t* sdoff = ws + L.o_sdoff;
  int32_t* ssrc = ws + L.o_ssrc;
  int32_t* srows = ws + L.o_srows;
  int32_t* sunit = ws + L.o_sunit;
  int* s_nrsegs = gseg;   // one LDS word (the per-group table is not needed)
  if (tid == 0) *s_nrsegs = -1;
  __syncthreads();
  const int NS = scan_items(
      B, starts_segment,
      [&](int b, int pre) {
        if (starts_segment(b)) sfirst[pre] = b;
        if (b == n_remote) *s_nrsegs = pre;   // the first local band starts a segment
      },
      sh);
  const int n_rsegs = (*s_nrsegs >= 0) ? *s_nrsegs : NS;
  for (int i = tid; i < NS; i += nt) {
    const int b0 = sfirst[i];
    const int b1 = (i + 1 < NS) ? sfirst[i + 1] : B;
    int rows = 0;
    for (int b = b0; b < b1; ++b) rows += bval[b];
    snb[i] = b1 - b0;
    sdst[i] = bdst[b0];
    sdoff[i] = bdoff[b0];
    ssrc[i] = bsrc[b0];
    srows[i] = rows;
  }
  __syncthreads();   // srows is read back by the scan
  const int U = scan_items(
      NS, [&](int i) { return units_of(srows[i]); }, [&](int i, int pre) { sunit[i] = pre; }, sh);
  if (tid == 0) sunit[NS] = U;

  // (h) padding entries of src_index: the tail of every remote group
  int32_t* src = ws + L.o_src;
  // one wavefront per group, its lanes over the group's (< tb) pad rows
  {
    const int wv = tid >> 6, nwv = nt >> 6, ln = tid & 63;
    for (int gi = wv; gi < NGR; gi += nwv) {
      int e, o;
      group_eo(gi, e, o);
      const int n = c[e * W + o];
      const int padded = ((n + tb - 1) / tb) * tb;
      const int row0 = rowoff[e] + grp[e * W + o];
      for (int q = n + ln; q < padded; q += 64) src[row0 + q] = -1;
    }
  }

  // (i) gate/up m-tiles: every X_e cut into kGuBM-row tiles, experts in order
  int32_t* mt_row = ws + L.o_gumt_row;
  int32_t* mt_exp = ws + L.o_gumt_exp;
  const int NMT = scan_items(
      E_l, [&](int q) { return (me[order[q]] + kGuBM - 1) / kGuBM; },
      [&](int q, int pre) {
        const int e = order[q];
        const int n = (me[e] + kGuBM - 1) / kGuBM;
        for (int i = 0; i < n; ++i) {
          mt_row[pre + i] = rowoff[e] + i * kGuBM;
          mt_exp[pre + i] = e;
        }
      },
      sh);

  // (j) down m-tiles, when tb_M divides 256: the runs of row-contiguous
  //     bands in S order -- the remote bands of each expert (its remote
  //     groups follow one another at the start of X_e), then the local bands
  //     of each expert -- cut into tiles of at most dn_merge bands
  int NDT = B * L.dn_sub;
  int* s_ndt_r = gunit;   // one LDS word: down row tiles of the remote runs
  if (tid == 0) *s_ndt_r = n_remote * L.dn_sub;
  __syncthreads();
  if (L.dn_merge > 0) {
    const int P = L.dn_merge;
    int32_t* dt_row = ws + L.o_dnt_row;
    int32_t* dt_exp = ws + L.o_dnt_exp;
    int32_t* dt_band = ws + L.o_dnt_band;
    int32_t* dt_nb = ws + L.o_dnt_nb;
    auto run_of = [&](int q, int& e, int& first, int& nb, int& row0) {
      if (q < E_l) {
        e = order[q];
        first = gstart[q * (W - 1)];   // with W == 1 there are no remote bands
        nb = rb[e];
        row0 = rowoff[e];
      } else {
        e = q - E_l;
        first = gstart[NGR + e];
        nb = (c[e * W + r] + tb - 1) / tb;
        row0 = rowoff[e] + grp[e * W + r];
      }
    };
    NDT = scan_items(
        2 * E_l,
        [&](int q) {
          int e, first, nb, row0;
          run_of(q, e, first, nb, row0);
          return (nb + P - 1) / P;
        },
        [&](int q, int pre) {
          if (q == E_l) *s_ndt_r = pre;   // the remote runs come first
          int e, first, nb, row0;
          run_of(q, e, first, nb, row0);
          for (int j = 0; j * P < nb; ++j) {
            dt_row[pre + j] = row0 + j * P * tb;
            dt_exp[pre + j] = e;
            dt_band[pre + j] = first + j * P;
            dt_nb[pre + j] = min(P, nb - j * P);
          }
        },
        sh);
  }

  // results used by later kernels and by inspection
  for (int i = tid; i < EW; i += nt) {
    ws[L.o_c + i] = c[i];
    ws[L.o_grp + i] = grp[i];
    ws[L.o_base + i] = base[i];
  }
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
    hdr[H_DN_MT_R] = *s_ndt_r;
  }
}

// in-wave stable rank of `v` among lanes holding the same value (v >= 0);
// the lowest lane of each value writes the wave's count into cnt[v]
__device__ __forceinline__ int wave_match_rank(int v, int* cnt) {
  const int lane = threadIdx.x & 63;
  uint64_t todo = __ballot(v >= 0);
  int rank = 0;
  while (todo) {
    const int leader = __ffsll((long long)todo) - 1;
    const int lv = __shfl(v, leader, 64);
    const uint64_t m = __ballot(v == lv);
    if (v == lv) rank = __popcll(m & lanes_below(lane));
    if (lane == leader) cnt[lv] = __popcll(m);
    todo &= ~m;
  }
  return rank;
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
  const int32_t* bp = ws + L.o_bp + (int64_t)b * (E_l + 1);
  const int recv_base = ws[L.o_brecv + b];
  int32_t* src = ws + L.o_src;
  const int32_t* bpr = ws + L.o_bpr + (int64_t)(b - L.blk_off[L.r]) * E;
  const int32_t* baser = ws + L.o_baser;
  int32_t* pos = ws + L.o_pos;
  const int lo = L.r * E_l;
  for (int p_base = p0; p_base < p1; p_base += blockDim.x) {
    const int p = p_base + tid;
    const int g = (p < p1) ? topk[p] : -1;
    const int e = (g >= lo && g < lo + E_l) ? g - lo : -1;
    const int re = wave_match_rank(e, wc + w * NX);
    const int rl = wave_match_rank(e >= 0 ? E_l : -1, wc + w * NX);
    int rg = 0;
    if (own) rg = wave_match_rank((g >= 0 && g < E) ? g : -1, wc_g + w * E);
    __syncthreads();
    if (e >= 0) {
      int rank_e = run[e] + re, rank_l = run[E_l] + rl;
      for (int x = 0; x < w; ++x) { rank_e += wc[x * NX + e]; rank_l += wc[x * NX + E_l]; }
      const int dest = rowoff[e] + grp[e * W + o] + bp[e] + rank_e;
      const int i = recv_base + rank_l;
      if (dest < L.rows_cap && i < L.R) src[dest] = i;
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

__global__ __launch_bounds__(256) void plan_gather_kernel(PlanLayout L, const int32_t* __restrict__ ws,
                                                         const uint4* __restrict__ x_recv,
                                                         uint4* __restrict__ x_layout) {
  const int32_t* hdr = ws + L.o_hdr;
  if (hdr[H_ERROR] != 0) return;
  const int M = hdr[H_M];
  const int32_t* src = ws + L.o_src;
  const int lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;
  const int64_t vec = L.d / 8;  // 16-byte vectors per row
  for (int row = blockIdx.x * wpb + (threadIdx.x >> 6); row < M; row += gridDim.x * wpb) {
    const int s = src[row];
    uint4* dst = x_layout + (int64_t)row * vec;
    if (s >= 0) {
      const uint4* sp = x_recv + (int64_t)s * vec;
      for (int64_t v = lane; v < vec; v += 64) dst[v] = sp[v];
    } else {
      const uint4 z = make_uint4(0, 0, 0, 0);
      for (int64_t v = lane; v < vec; v += 64) dst[v] = z;
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
  const int words = build_lds_words(L.W, L.E_l, L.E) + (L.build_stage ? L.NB * (L.E_l + 2) + L.NB_r * L.E : 0);
  hipLaunchKernelGGL(plan_build_kernel, dim3(1), dim3(kBuildThreads), (size_t)words * sizeof(int), s, L, ws);
  if (L.NB > 0) {
    const int nw = kPlanThreads / 64;
    const size_t sh_place = (size_t)((L.E_l + 1) * (nw + 1) + L.E * (nw + 1)) * sizeof(int);
    hipLaunchKernelGGL(plan_place_kernel, dim3(L.NB), dim3(kPlanThreads), sh_place, s, L, topk, ws);
  }
  const int rows_per_block = 4;
  int grid = (L.rows_cap + rows_per_block - 1) / rows_per_block;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(plan_gather_kernel, dim3(grid), dim3(256), 0, s, L, (const int32_t*)ws,
                     (const uint4*)x_recv, (uint4*)x_layout);
  return hipGetLastError();
}

}  // namespace moe
