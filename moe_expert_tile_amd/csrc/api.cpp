// C ABI of libmoe.so (declared in include/moe.h): host-side validation,
// workspace layout, CU-partitioned streams and launch orchestration.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string.h>

#include "moe.h"
#include "moe_internal.h"

namespace moe {

namespace {

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int valid_shape(const moe_shape* s) {
  if (!s || !s->tokens) return MOE_EINVAL;
  if (s->world < 1 || s->world > kMaxWorld) return MOE_EINVAL;
  if (s->rank < 0 || s->rank >= s->world) return MOE_EINVAL;
  if (s->experts_per_rank < 1 || (int64_t)s->experts_per_rank * s->world > 1024) return MOE_EINVAL;
  const int E = s->experts_per_rank * s->world;
  if (s->top_k < 1 || s->top_k > 32 || s->top_k > E) return MOE_EINVAL;
  if (s->hidden < 256 || s->hidden % 256 != 0 || s->hidden > 65536) return MOE_EINVAL;
  if (s->ffn < 128 || s->ffn % 128 != 0 || s->ffn > 65536) return MOE_EINVAL;
  // the GEMMs address one expert's weights with 32-bit byte offsets
  if ((int64_t)s->ffn * s->hidden >= (1ll << 30)) return MOE_EINVAL;
  if (s->tb_m < 32 || s->tb_m > 256 || s->tb_m % 32 != 0) return MOE_EINVAL;
  if (s->mgb < 1 || s->mgb > 64) return MOE_EINVAL;
  int64_t pairs = 0;
  for (int o = 0; o < s->world; ++o) {
    if (s->tokens[o] < 0) return MOE_EINVAL;
    pairs += (int64_t)s->tokens[o] * s->top_k;
  }
  if (pairs > (1ll << 30)) return MOE_EINVAL;
  if (s->recv_rows < 0 || s->recv_rows > pairs) return MOE_EINVAL;
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

bool make_layout(int W, int r, int E_l, int k, int d, int f, int tb_m, int mgb, const int32_t* tokens, int64_t R,
                 PlanLayout* L) {
  memset(L, 0, sizeof(*L));
  L->W = W; L->r = r; L->E_l = E_l; L->E = W * E_l; L->k = k; L->d = d; L->f = f;
  L->tb_m = tb_m; L->mgb = mgb; L->R = (int)R;
  const int64_t rows_cap = R + (int64_t)E_l * (W - 1) * (tb_m - 1);
  if (rows_cap > (1ll << 30)) return false;
  L->rows_cap = (int)rows_cap;
  L->bands_cap = (int)(rows_cap / tb_m + (int64_t)E_l * W);
  L->T_r = tokens[r];
  int pair = 0, blk = 0, tok = 0;
  for (int o = 0; o < W; ++o) {
    L->pair_off[o] = pair;
    L->blk_off[o] = blk;
    L->tok_off[o] = tok;
    const int p = tokens[o] * k;
    pair += p;
    blk += (p + kPairsPerBlock - 1) / kPairsPerBlock;
    tok += tokens[o];
  }
  L->pair_off[W] = pair;
  L->blk_off[W] = blk;
  L->tok_off[W] = tok;
  L->NB = blk;
  L->NB_r = L->blk_off[r + 1] - L->blk_off[r];
  // down GEMM: the gate/up GEMM's 256-row tiles of compacted rows; a pair of
  // flags (band head, band tail) per band and column tile
  L->dn_ntn = d / kDnBN;
  L->dn_tpb = L->dn_ntn;
  L->gu_ntn = f / (kGuBN / 2);
  L->gu_mt_cap = (int)(rows_cap / kGuBM + E_l + 1);
  L->band_lds = 0;  // decided at launch, against the device's LDS limit
  // the planner's divisors: row counts (below 2^31), band and group indices
  L->div_tb = make_fastdiv(tb_m, 31);
  L->div_mgb = make_fastdiv(mgb, 31);
  L->div_wm1 = make_fastdiv(W > 1 ? W - 1 : 1, 31);
  L->div_hb = make_fastdiv(E_l + 2, 31);
  L->div_w = make_fastdiv(W, 31);
  L->div_el = make_fastdiv(E_l, 31);

  int64_t off = 0;
  auto take = [&](int64_t n) {
    const int64_t at = off;
    off += round_up(n > 0 ? n : 1, 64);  // 256-byte aligned pieces
    return at;
  };
  const int64_t EW = (int64_t)E_l * W, B = L->bands_cap;
  L->o_hdr = take(H_WORDS);
  L->o_c = take(EW);
  L->o_low = take(W);
  L->o_grp = take(EW);
  L->o_me = take(E_l);
  L->o_rowoff = take(E_l + 1);
  L->o_rb = take(E_l);
  L->o_order = take(E_l);
  L->o_base = take(EW);
  L->o_bexp = take(B); L->o_bdst = take(B); L->o_bsrc = take(B); L->o_bdoff = take(B); L->o_bval = take(B);
  L->o_sfirst = take(B); L->o_snb = take(B); L->o_sdst = take(B); L->o_sdoff = take(B); L->o_ssrc = take(B);
  L->o_srows = take(B); L->o_sunit = take(B + 1);
  L->o_src = take(rows_cap);
  L->o_pos = take((int64_t)L->T_r * k);
  L->o_bh = take((int64_t)L->NB * (E_l + 2));
  L->o_bhr = take((int64_t)L->NB_r * L->E);
  L->o_obase = take(W + 1);
  L->o_grow = take(EW);
  L->o_gcrow = take(EW);
  L->o_btmp = take(4 * (B + 1));
  L->o_gband = take(EW);
  L->o_gumt_row = take(L->gu_mt_cap);
  L->o_gumt_exp = take(L->gu_mt_cap);
  L->o_dnt_row = take(L->gu_mt_cap); L->o_dnt_exp = take(L->gu_mt_cap);
  L->o_crowoff = take(E_l + 1);
  L->o_ccum = take(EW);
  L->o_bcrow = take(B);
  L->o_cmprow = take(R);
  L->o_cmpsrc = take(R);
  // stream-K partial-sum slots: as many as the larger GEMM can split.  A
  // split happens only for K >= kMinSkKTOneRound steps (kMinSkKT behind full
  // rounds); its tiles are at most 3/4 of a round (half a round when only
  // the one-round rule applies), and their K steps are cut into at most
  // min(G, steps / kMinSkSteps) pieces, two slots each (a piece may close
  // one tile and open the next).
  const int64_t gu_tiles_max = (int64_t)L->gu_mt_cap * L->gu_ntn;
  const int64_t dn_tiles_max = (int64_t)L->gu_mt_cap * L->dn_ntn;
  auto sk_need = [](int64_t tiles_max, int KT) -> int64_t {
    if (KT < kMinSkKTOneRound || tiles_max <= 0) return 0;
    const int64_t split_max = KT >= kMinSkKT ? 3 * kMaxProducers / 4 : kMaxProducers / 2;
    const int64_t tiles = std::min(tiles_max, split_max);
    return 2 * std::min<int64_t>(kMaxProducers, tiles * KT / kMinSkSteps);
  };
  L->sk_slots = (int)std::max(sk_need(gu_tiles_max, d / kGuBK), sk_need(dn_tiles_max, f / kDnBK));
  L->o_link = take(2 * kMaxWorld);             // uint64 per destination
  L->o_gready = take(2 * EW);                  // uint64 per (expert, destination) group
  L->o_skc = take(2 * kMaxProducers * 2);
  L->o_skp = take((int64_t)L->sk_slots * 256 * 256);
  L->total_words = off;
  return true;
}

// --- per-device cache: compute units and LDS limit ---
namespace {

struct DeviceState {
  bool init = false;
  int cus = 0;
  int lds_per_block = 0;
};
constexpr int kMaxDevices = 16;
DeviceState g_dev[kMaxDevices];
std::mutex g_mu;

int current_device(int* dev) {
  if (hipGetDevice(dev) != hipSuccess) return MOE_EUNSUPPORTED;
  if (*dev < 0 || *dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int device_cus(int dev) {
  DeviceState& st = g_dev[dev];
  if (!st.init) {
    int n = 0, lds = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
    st.cus = n;
    st.lds_per_block = lds;
    st.init = true;
  }
  return st.cus;
}

int check_gfx950(int dev) {
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return MOE_EUNSUPPORTED;
  if (strncmp(p.gcnArchName, "gfx950", 6) != 0) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int prepare(int* dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  int rc = current_device(dev);
  if (rc) return rc;
  DeviceState& st = g_dev[*dev];
  if (!st.init) {
    rc = check_gfx950(*dev);
    if (rc) return rc;
    if (device_cus(*dev) <= 0) return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Grid of the standalone consumer: one workgroup per copy unit.  The remote
// units are known only on the device; Σ_seg ceil(bytes_seg / chunk) is at
// most R·d·2 / chunk plus one per segment (segments <= bands), and the
// workgroups past the true count return at once.
int consumer_grid(const PlanLayout& L) {
  const int64_t bound = (int64_t)L.R * L.d * 2 / kCopyChunk + L.bands_cap + 1;
  return (int)std::max<int64_t>(1, std::min<int64_t>(bound, 65535));
}

void record(void* ev, hipStream_t s) {
  if (ev) (void)hipEventRecord((hipEvent_t)ev, s);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ECAPACITY: return "capacity exceeded";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_ETIMEOUT: return "consumer wait timed out";
    case MOE_EROUTING: return "routing inconsistent (expert id out of range or received-row count mismatch)";
    case MOE_EUNSUPPORTED: return "no gfx950 device";
    default: return "unknown status";
  }
}

int moe_query_sizes(const moe_shape* s, moe_sizes* out) {
  int rc = valid_shape(s);
  if (rc) return rc;
  if (!out) return MOE_EINVAL;
  PlanLayout L;
  if (!make_layout(s->world, s->rank, s->experts_per_rank, s->top_k, s->hidden, s->ffn, s->tb_m, s->mgb, s->tokens,
                   s->recv_rows, &L))
    return MOE_ECAPACITY;
  out->plan_bytes = (size_t)L.total_words * 4;
  out->rows_cap = L.rows_cap;
  out->bands_cap = L.bands_cap;
  out->flags_count = 2 * (int64_t)L.bands_cap * L.dn_tpb;
  out->recv_rows_self = (int64_t)L.T_r * L.k;
  return MOE_OK;
}

int moe_plan_offsets(const moe_shape* s, moe_plan_view* v) {
  int rc = valid_shape(s);
  if (rc) return rc;
  if (!v) return MOE_EINVAL;
  PlanLayout L;
  if (!make_layout(s->world, s->rank, s->experts_per_rank, s->top_k, s->hidden, s->ffn, s->tb_m, s->mgb, s->tokens,
                   s->recv_rows, &L))
    return MOE_ECAPACITY;
  v->hdr = L.o_hdr * 4; v->c = L.o_c * 4; v->grp_off = L.o_grp * 4; v->m_e = L.o_me * 4;
  v->row_off = L.o_rowoff * 4; v->rb = L.o_rb * 4; v->order = L.o_order * 4; v->base = L.o_base * 4;
  v->band_expert = L.o_bexp * 4; v->band_dst = L.o_bdst * 4; v->band_src_row = L.o_bsrc * 4;
  v->band_dst_off = L.o_bdoff * 4; v->band_valid = L.o_bval * 4;
  v->seg_first = L.o_sfirst * 4; v->seg_nbands = L.o_snb * 4; v->seg_dst = L.o_sdst * 4;
  v->seg_dst_off = L.o_sdoff * 4; v->seg_src_row = L.o_ssrc * 4; v->seg_rows = L.o_srows * 4;
  v->seg_unit = L.o_sunit * 4; v->src_index = L.o_src * 4; v->pos = L.o_pos * 4;
  v->gu_tile_row = L.o_gumt_row * 4; v->gu_tile_expert = L.o_gumt_exp * 4;
  v->dn_tile_row = L.o_dnt_row * 4; v->dn_tile_expert = L.o_dnt_exp * 4;
  v->grp_band = L.o_gband * 4;
  v->sk_counters = L.o_skc * 4; v->sk_counters_count = 2 * kMaxProducers;
  v->crow_off = L.o_crowoff * 4; v->grp_crow = L.o_ccum * 4; v->band_crow = L.o_bcrow * 4;
  v->cmp_row = L.o_cmprow * 4; v->cmp_src = L.o_cmpsrc * 4;
  return MOE_OK;
}

int moe_plan(const moe_shape* s, const int32_t* topk_ids, const uint16_t* x_recv, void* plan_ws,
             uint16_t* x_layout, void* stream) {
  int rc = valid_shape(s);
  if (rc) return rc;
  int64_t pairs = 0;
  for (int o = 0; o < s->world; ++o) pairs += (int64_t)s->tokens[o] * s->top_k;
  if (!plan_ws || !aligned(plan_ws, 256)) return MOE_EINVAL;
  if (pairs > 0 && (!topk_ids || !aligned(topk_ids, 4))) return MOE_EINVAL;
  if (s->recv_rows > 0 && (!x_recv || !aligned(x_recv, 16))) return MOE_EINVAL;
  if (x_layout && !aligned(x_layout, 16)) return MOE_EINVAL;   // NULL: metadata only
  PlanLayout L;
  if (!make_layout(s->world, s->rank, s->experts_per_rank, s->top_k, s->hidden, s->ffn, s->tb_m, s->mgb, s->tokens,
                   s->recv_rows, &L))
    return MOE_ECAPACITY;
  int dev;
  rc = prepare(&dev);
  if (rc) return rc;
  // the plan builder keeps its per-band tables in LDS when they fit the
  // device's per-workgroup LDS (every shape here but the largest)
  const int64_t lds_cap = std::min<int64_t>(g_dev[dev].lds_per_block, kBuildLdsBytes);
  L.band_lds = (int64_t)build_lds(L.W, L.E_l, L.bands_cap, true).total * 4 <= lds_cap;
  return hip_rc(launch_plan(L, topk_ids, x_recv, (int32_t*)plan_ws, x_layout, (hipStream_t)stream));
}

}  // extern "C"

namespace moe {

// moe_expert_combine with its kernels' scratch either in the plan workspace
// (get_scratch == nullptr) or where get_scratch(device, &sc) puts it; then
// the counters are cleared first, since that scratch outlives the call.
int combine_impl(const moe_shape* s, const void* plan_ws, const uint16_t* x_layout, const uint16_t* w_gate_up,
                 const uint16_t* w_down, uint16_t* h, uint16_t* y, uint32_t* flags, uint32_t epoch,
                 uint16_t* const* recv, const moe_combine_opts* opts, void* stream,
                 int (*get_scratch)(int dev, Scratch* out)) {
  int rc = valid_shape(s);
  if (rc) return rc;
  moe_combine_opts o;
  memset(&o, 0, sizeof(o));
  if (opts) o = *opts;
  if (o.mode < MOE_MODE_OVERLAP || o.mode > MOE_MODE_COPY_ROWS) return MOE_EINVAL;
  if (o.consumer_cus == 0) o.consumer_cus = 16;
  if (o.consumer_cus < 8 || o.consumer_cus > 128 || o.consumer_cus % 8 != 0) return MOE_EINVAL;
  if (o.consumer_blocks < 0 || o.consumer_blocks > 65536) return MOE_EINVAL;
  // OVERLAP: each consumer workgroup must have a reserved CU of its own
  if (o.mode == MOE_MODE_OVERLAP && o.consumer_blocks > o.consumer_cus) return MOE_EINVAL;
  if (o.spin_timeout_ns < 0) return MOE_EINVAL;
  if (o.link_mbps < 0 || (o.link_mbps > 0 && o.link_mbps < 1000)) return MOE_EINVAL;
  if (o.signal != MOE_SIGNAL_TILE && o.signal != MOE_SIGNAL_GROUP) return MOE_EINVAL;
  if (o.signal == MOE_SIGNAL_GROUP && o.mode == MOE_MODE_COPY_ROWS) return MOE_EINVAL;
  if (epoch == 0) return MOE_EINVAL;
  if (!plan_ws || !aligned(plan_ws, 256)) return MOE_EINVAL;
  const bool compute = (o.mode != MOE_MODE_COPY_ONLY && o.mode != MOE_MODE_COPY_ROWS);
  // A rows of the gate/up GEMM: the materialized layout, or gathered from
  // x_recv through src_index (padding rows read past the buffer's bound)
  const uint16_t* a_rows = x_layout;
  bool gathered = false;
  if (compute) {
    if (!x_layout) {
      const int64_t a_bytes = s->recv_rows * (int64_t)s->hidden * 2;
      if (a_bytes >= (1ll << 31)) return MOE_EINVAL;
      if (s->recv_rows > 0 && (!o.x_recv || !aligned(o.x_recv, 16))) return MOE_EINVAL;
      a_rows = (const uint16_t*)o.x_recv;
      gathered = true;
    } else if (!aligned(x_layout, 16)) {
      return MOE_EINVAL;
    }
    if (!w_gate_up || !aligned(w_gate_up, 16) || !w_down || !aligned(w_down, 16) || !h || !aligned(h, 16))
      return MOE_EINVAL;
  }
  if (!y || !aligned(y, 16) || !flags || !aligned(flags, 4) || !recv) return MOE_EINVAL;
  RecvPtrs rp;
  memset(&rp, 0, sizeof(rp));
  for (int i = 0; i < s->world; ++i) {
    if (s->tokens[i] > 0 && (!recv[i] || !aligned(recv[i], 16))) return MOE_EINVAL;
    rp.p[i] = recv[i];
  }
  PlanLayout L;
  if (!make_layout(s->world, s->rank, s->experts_per_rank, s->top_k, s->hidden, s->ffn, s->tb_m, s->mgb, s->tokens,
                   s->recv_rows, &L))
    return MOE_ECAPACITY;
  int dev;
  rc = prepare(&dev);
  if (rc) return rc;
  const int cus = g_dev[dev].cus;
  const int64_t timeout = (o.spin_timeout_ns ? o.spin_timeout_ns : 2000000000ll) / 10;  // 100 MHz ticks
  const hipStream_t st = (hipStream_t)stream;
  const int32_t* ws = (const int32_t*)plan_ws;
  int32_t* ws_rw = (int32_t*)plan_ws;
  int full_grid = std::min(cus, kMaxProducers);
  full_grid -= full_grid % 8;
  if (full_grid < 8) full_grid = 8;
  Scratch sc;
  if (get_scratch) {
    rc = get_scratch(dev, &sc);
    if (rc) return rc;
  } else {
    sc.sk_part = (float*)(ws_rw + L.o_skp);
    sc.sk_ctr = (uint64_t*)(ws_rw + L.o_skc);
    sc.claim = ws_rw + L.o_hdr + H_CLAIM;
    sc.link_free = (uint64_t*)(ws_rw + L.o_link);
    sc.gready = (uint64_t*)(ws_rw + L.o_gready);
    sc.sk_slots = L.sk_slots;
  }
  CopyCtl cc;
  cc.timeout = timeout;
  cc.link_mbps = (uint32_t)o.link_mbps;
  cc.signal = o.signal;
  cc.link_free = sc.link_free;
  cc.gready = sc.gready;

  if (o.mode == MOE_MODE_COPY_ROWS) {
    record(o.events[4], st);
    rc = hip_rc(launch_consumer_rows(L, ws_rw, y, flags, epoch, rp, timeout, st));
    record(o.events[5], st);
    return rc;
  }
  if (o.mode == MOE_MODE_COPY_ONLY) {
    record(o.events[4], st);
    rc = hip_rc(launch_consumer(L, ws_rw, y, flags, epoch, rp, cc, o.consumer_blocks ? o.consumer_blocks : consumer_grid(L),
                                st));
    record(o.events[5], st);
    return rc;
  }
  if (get_scratch) {
    rc = hip_rc(launch_clear_counters(sc, st));
    if (rc) return rc;
  }
  record(o.events[0], st);
  rc = hip_rc(launch_gateup(L, ws_rw, sc, a_rows, gathered, w_gate_up, h, epoch, full_grid, st));
  record(o.events[1], st);
  if (rc) return rc;
  if (o.mode == MOE_MODE_SERIAL) {
    record(o.events[2], st);
    rc = hip_rc(launch_down(L, ws_rw, sc, h, w_down, y, flags, epoch, rp, cc, full_grid, full_grid, st));
    record(o.events[3], st);
    if (rc) return rc;
    record(o.events[4], st);
    rc = hip_rc(launch_consumer(L, ws_rw, y, flags, epoch, rp, cc, o.consumer_blocks ? o.consumer_blocks : consumer_grid(L),
                                st));
    record(o.events[5], st);
    return rc;
  }
  // OVERLAP (§5.3): one launch on the caller's stream; the first n_prod
  // workgroups run the down GEMM, the last consumer_cus (one per CU, as the
  // GEMM's LDS footprint leaves room for one workgroup per CU) consume
  if (o.consumer_cus >= cus) return MOE_EINVAL;
  int n_prod = std::min(cus - o.consumer_cus, kMaxProducers);
  n_prod -= n_prod % 8;
  const int n_cons = o.consumer_blocks ? o.consumer_blocks : o.consumer_cus;
  record(o.events[2], st);
  record(o.events[4], st);
  rc = hip_rc(launch_down(L, ws_rw, sc, h, w_down, y, flags, epoch, rp, cc, n_prod, n_prod + n_cons, st));
  record(o.events[3], st);
  record(o.events[5], st);
  return rc;
}

}  // namespace moe

extern "C" {

int moe_expert_combine(const moe_shape* s, const void* plan_ws, const uint16_t* x_layout, const uint16_t* w_gate_up,
                       const uint16_t* w_down, uint16_t* h, uint16_t* y, uint32_t* flags, uint32_t epoch,
                       uint16_t* const* recv, const moe_combine_opts* opts, void* stream) {
  return combine_impl(s, plan_ws, x_layout, w_gate_up, w_down, h, y, flags, epoch, recv, opts, stream, nullptr);
}

int moe_scale(const moe_shape* s, const void* plan_ws, const uint16_t* recv_self, const float* topk_w, uint16_t* out,
              void* stream) {
  int rc = valid_shape(s);
  if (rc) return rc;
  if (!plan_ws || !aligned(plan_ws, 256)) return MOE_EINVAL;
  const int T = s->tokens[s->rank];
  if (T > 0 && (!recv_self || !aligned(recv_self, 16) || !topk_w || !aligned(topk_w, 4) || !out ||
                !aligned(out, 16)))
    return MOE_EINVAL;
  PlanLayout L;
  if (!make_layout(s->world, s->rank, s->experts_per_rank, s->top_k, s->hidden, s->ffn, s->tb_m, s->mgb, s->tokens,
                   s->recv_rows, &L))
    return MOE_ECAPACITY;
  int dev;
  rc = prepare(&dev);
  if (rc) return rc;
  return hip_rc(launch_scale(L, (const int32_t*)plan_ws, recv_self, topk_w, out, (hipStream_t)stream));
}

int moe_device_status(const void* plan_ws, void* stream) {
  if (!plan_ws || !aligned(plan_ws, 256)) return MOE_EINVAL;
  const hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_EHIP;
  int32_t word = 0;
  if (hipMemcpy(&word, plan_ws, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return MOE_EHIP;
  return word;
}

int moe_device_cus(void) {
  int dev;
  if (prepare(&dev) != MOE_OK) return 0;
  return g_dev[dev].cus;
}

}  // extern "C"
