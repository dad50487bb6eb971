// Expert FFN as grouped bf16 MFMA GEMMs over the owner-aligned layout.
//
// Tile-signal notes ("MoE 计算-通信细粒度重叠：用 Tile 级信号把 All-to-All 藏在 GEMM 背后"):
// §5.1 — one persistent GEMM over all local experts; workgroup i takes tiles
// i, i+g, i+2g, ... in schedule order; the per-expert operand pointers are
// looked up per tile; after a tile is stored and made globally visible a
// per-tile ready flag is set.  §2.3 — the epilogue is where the flag goes.
//
// gfx950 design (not the pages' CUTLASS one):
//   * v_mfma_f32_32x32x16_bf16, fp32 accumulation, 64-wide wavefronts;
//     8 wavefronts per workgroup (2 per SIMD), each owning a WM x WN register
//     tile of a 256 x 256 output tile (gate/up: 128 gate + 128 up columns
//     of the same indices, so SwiGLU is fused in the epilogue).
//   * The MFMA's first operand is the weight tile (rows = output columns n),
//     the second the activation tile (rows = output rows m), so each lane ends
//     with 4 consecutive output columns per accumulator quad, and the SwiGLU
//     gate/up pair of a column sits in one lane.
//   * K steps of 64: both operands are K-contiguous in HBM, copied straight
//     into LDS with 16-byte buffer loads (no staging registers) into one ring
//     per operand, 16-byte chunks XOR-swizzled so that the ds_read_b128
//     operand fetches are bank-conflict free on the 64-bank LDS.
//   * Epilogues: gate/up stores h from registers; the down GEMM stages its
//     tile through LDS and writes whole lines with device-scope
//     (write-through) stores, and sets the tile's flags once they are
//     acknowledged (at the next tile's prologue).
//   * Persistent grid (a multiple of 8 workgroups).  Workgroup w runs on XCD
//     w mod 8; it takes slot (w mod 8) * (G/8) + w/8 of every round of G
//     tiles, so each XCD works on a contiguous run of the tile order, and the
//     two-level tile order (decode_tile) makes that run a block of 8 row
//     tiles x 4 column tiles whose operands share the XCD's L2.  Fewer tiles
//     than workgroups go round-robin over the XCDs instead.
#include <type_traits>

#include "consume.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Tile shapes (compile-time; the defaults are the measured best on MI355X).
#ifndef MOE_XCD_ROWS
// XCDs sharing a weight block in the two-level tile order (1, 2, 4, 8), for
// the gate/up GEMM.  Measured: the gate/up GEMMs are within noise of 1; 8
// is slower on the DeepSeek-like share.
#define MOE_XCD_ROWS 2
#endif
#ifndef MOE_XCD_ROWS_DN
// The same for the down GEMM.  Measured over an earlier band-packed tiling
// (same box, serial mode, two passes): 1 takes the DeepSeek-like down GEMM
// from 1663-1693 to 1621-1636 us and leaves the Mixtral- and Qwen3-like ones
// within noise; 4 and 8 are 2-4% slower there, and per-XCD blocks of 4 x 8,
// 2 x 16, 16 x 2 or 32 x 1 tiles are no better than 8 x 4.  Over the
// current tiles 2 is 0.6-3% slower than 1 (DeepSeek- and Qwen3-like).
#define MOE_XCD_ROWS_DN 1
#endif
#ifndef MOE_GU_WAVES_M
#define MOE_GU_WAVES_M 4
#endif
#ifndef MOE_GU_WAVES_N
#define MOE_GU_WAVES_N 2
#endif
#ifndef MOE_DN_WAVES_M
#define MOE_DN_WAVES_M 2
#endif
#ifndef MOE_DN_WAVES_N
#define MOE_DN_WAVES_N 4
#endif
#ifndef MOE_GU_BK
#define MOE_GU_BK 64
#endif
#ifndef MOE_GU_SA
#define MOE_GU_SA 2
#endif
#ifndef MOE_GU_SB
#define MOE_GU_SB 2
#endif
#ifndef MOE_DN_BK
#define MOE_DN_BK 64
#endif
#ifndef MOE_DN_SA
#define MOE_DN_SA 2
#endif
#ifndef MOE_DN_SB
#define MOE_DN_SB 2
#endif
#ifndef MOE_STORE_AUX
// cache-policy bits of the down GEMM's output stores: sc1 (bit 4), device
// scope, written through this XCD's L2; the flag publication relies on it
// (measured 3-20% faster than the default policy even with a release fence)
#define MOE_STORE_AUX 16
#endif
#ifndef MOE_LOAD_AUX
#define MOE_LOAD_AUX 0   // cache-policy bits of the operand loads (default policy measured best)
#endif
constexpr int kDeviceScope = 16;   // sc1 cache-policy bit: device scope, written through the XCD's L2
constexpr int kXcdRowsGu = MOE_XCD_ROWS;
constexpr int kXcdRowsDn = MOE_XCD_ROWS_DN;
static_assert(kXcdRowsGu == 1 || kXcdRowsGu == 2 || kXcdRowsGu == 4 || kXcdRowsGu == 8, "XCD rows");
static_assert(kXcdRowsDn == 1 || kXcdRowsDn == 2 || kXcdRowsDn == 4 || kXcdRowsDn == 8, "XCD rows");

// BM x BN output tile, WAVES_M x WAVES_N wavefronts, K step BK; the A and B
// operands have their own global -> LDS rings, SA and SB stages deep (2 or
// 3).  An LDS row holds BK bf16 (BK/8 chunks of 16 bytes); chunks are
// XOR-swizzled so that any 16 lanes reading 16 consecutive rows at the same
// logical chunk touch 16 distinct 16-byte bank groups of gfx950's 64-bank LDS
// (one ds_read_b128 phase).
template <int BM_, int BN_, int WAVES_M, int WAVES_N, int BK_, int SA_, int SB_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, SA = SA_, SB = SB_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int FM = WM / 32;
  static constexpr int FN = WN / 32;
  static constexpr int KK = BK / 16;            // MFMA k-steps per stage
  static constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row
  static constexpr int RPB = 1024 / (BK * 2);   // rows per 1 KB wave load
  static constexpr int R256 = 256 / (BK * 2);   // rows per 256-byte bank line
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BN * BK;
  static constexpr int LDS_ELEMS = SA * A_ELEMS + SB * B_ELEMS;
  static constexpr int LDS_BYTES = LDS_ELEMS * 2;
  static constexpr int A_LOADS = BM / RPB / NW;  // 1 KB wave loads per stage and wave
  static constexpr int B_LOADS = BN / RPB / NW;
  static constexpr int LPW = A_LOADS + B_LOADS;
  static constexpr int S_DEEP = SA > SB ? SA : SB;
  static constexpr int S_SHALLOW = SA < SB ? SA : SB;
  // loads of this wave still in flight at a K step's barrier (while a later
  // stage exists): the newest stage of every 3-deep ring
  static constexpr int DEEP_LOADS = (SA == 3 ? A_LOADS : 0) + (SB == 3 ? B_LOADS : 0);
  static_assert(NW == 4 || NW == 8, "four or eight wavefronts per workgroup");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "every wavefront loads both operands");
  static_assert(BM % (RPB * NW) == 0 && BN % (RPB * NW) == 0, "whole wave loads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(SA >= 2 && SA <= 3 && SB >= 2 && SB <= 3, "ring depths 2 or 3");
  static_assert(DEEP_LOADS <= 63, "vmcnt range");
  __device__ static int swz(int row, int c) { return c ^ ((row / R256) % CPR); }
};

struct GemmArgs {
  int32_t* ws;
  const uint16_t* a;      // activations [rows, K]
  const uint16_t* w;      // weights [E_l, N_total, K]
  uint16_t* out;          // [rows, out_cols]
  uint32_t* flags;
  uint32_t epoch;
  int K;                  // reduction length
  int out_cols;           // columns of `out`
  int w_rows;             // rows of one expert's weight matrix
  int half;               // SWIGLU: f (offset of the up rows); else 0
  int n_prod;             // producer workgroups (the rest of the grid consumes)
  CopyCtl cc;             // consumer: wait bound, link pacing, signal mode
  // gate/up: the table of A rows of the compacted rows (cmp_src into x_recv
  // when `gathered`, else cmp_row into the layout X); null for the down GEMM
  const int32_t* rows;
  int gathered;
  int64_t a_bytes;        // gathered: bytes of `a` (< 2^31)
  Scratch sc;             // stream-K partials and counters, copy-claim counters
};

__device__ __forceinline__ void stamp_max(int32_t* hdr, int word) {
  __hip_atomic_fetch_max((uint64_t*)(hdr + word), (uint64_t)wall_clock64(), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// K-step barriers wait for this wave's own outstanding global->LDS loads with
// the waitcnt builtin (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8): __syncthreads() would wait for every outstanding
// load (vmcnt(0)) and so drain the prefetch rings, and inline assembly would
// hide the wait from the compiler's own counter tracking.
__host__ __device__ constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4); }

// Workgroup barrier of a K step: this wavefront waits until at most `n` of
// its global->LDS loads are outstanding (n is 0 or one of the compile-time
// load counts) and its LDS reads are done, then all wavefronts meet.
template <class C>
__device__ __forceinline__ void stage_barrier(int n) {
  if (n == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  else if (n == C::A_LOADS) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(C::A_LOADS));
  else if (n == C::B_LOADS) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(C::B_LOADS));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(C::LPW));
  __builtin_amdgcn_s_barrier();
}

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x8, kSchedVmem = 0x10, kSchedDsRead = 0x100;

// Tile t of a (n_mt x n_nt) grid -> (mt, nt), in a two-level order.  A
// round of the persistent grid hands each XCD G/8 consecutive tiles; those
// form a block of SR row tiles x SC column tiles with SR * SC = G/8 when G/8
// factors so (8 x 4 for 32 producers per XCD, 6 x 5 for 30, 7 x 4 for 28;
// else 8 x 4, not aligned with the rounds), so a round's tiles on one XCD
// share SR + SC operand blocks in its L2.  The 8 XCDs' blocks form a chip
// block of SR*XR row tiles x SC*(8/XR) column tiles, so that XR XCDs read the
// same weight blocks (and 8/XR the same activation blocks) at the same time,
// which turns more of their L2 misses into Infinity Cache hits instead of
// HBM reads.  Chip blocks sweep the columns of a row group, row groups follow
// one another; ragged edges give smaller blocks.
__device__ __forceinline__ void xcd_block_shape(int per_xcd, int& SR, int& SC) {
  SR = 8;
  SC = 4;
  for (int sc = 8; sc >= 2; --sc) {
    if (per_xcd % sc == 0 && per_xcd / sc >= sc) {
      SR = per_xcd / sc;
      SC = sc;
      return;
    }
  }
}

template <int XR>
__device__ __forceinline__ void decode_tile(int t, int n_mt, int n_nt, int SR, int SC, int& mt, int& nt) {
  constexpr int XC = 8 / XR;
  const int BR = SR * XR, BC = SC * XC;
  const int full_rg = n_mt / BR;
  int rg, rr, t1;
  if (t < full_rg * BR * n_nt) {
    rg = t / (BR * n_nt);
    rr = BR;
    t1 = t - rg * BR * n_nt;
  } else {
    rg = full_rg;
    rr = n_mt - full_rg * BR;
    t1 = t - full_rg * BR * n_nt;
  }
  const int full_cb = n_nt / BC;
  int cb, cc, t2;
  if (t1 < full_cb * rr * BC) {
    cb = t1 / (rr * BC);
    cc = BC;
    t2 = t1 - cb * rr * BC;
  } else {
    cb = full_cb;
    cc = n_nt - full_cb * BC;
    t2 = t1 - full_cb * rr * BC;
  }
  // SR x SC blocks of the chip block, column blocks outer, rows fastest inside
  const int nsr = (rr + SR - 1) / SR, nsc = (cc + SC - 1) / SC;
  mt = rg * BR;
  nt = cb * BC;
  for (int sx = 0; sx < nsc; ++sx) {
    const int cw = min(SC, cc - SC * sx);
    for (int sr = 0; sr < nsr; ++sr) {
      const int rh = min(SR, rr - SR * sr);
      const int n = rh * cw;
      if (t2 < n) {
        mt += SR * sr + t2 % rh;
        nt += SC * sx + t2 / rh;
        return;
      }
      t2 -= n;
    }
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ float silu_f(float g) {
  // silu(g) = g / (1 + e^-g), e^-g = 2^(-g log2 e)
  return g / (1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

// Buffer resource word 3 for untyped (raw) buffer access on gfx9-family
// chips: data format 32, every other field zero.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufWord3);
}

// One operand's share of a stage: wave `wave` fills LDS rows [RPB q, RPB (q+1))
// for q = wave, wave + NW, ...; the lane byte offsets (from wave-uniform
// bases) carry the swizzled chunk, the K offset goes in the scalar offset.
// MUBUF loads with the LDS bit count only in vmcnt, so the LDS-read waits
// around them stay partial.
template <int NLOADS, int NW>
__device__ __forceinline__ void issue_operand(lds_void_t* dst, __amdgpu_buffer_rsrc_t rsrc,
                                              const uint32_t (&off)[NLOADS], int k0, int wave) {
  char* base = (char*)dst;
  const int koff = 2 * k0;
#pragma unroll
  for (int i = 0; i < NLOADS; ++i) {
    const int q = wave + i * NW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(base + q * 1024), 16, (int)off[i], koff, 0,
                                             MOE_LOAD_AUX);
  }
}

// The down GEMM's epilogue tables in LDS, past the operand rings (int
// words): per group k of the tile's expert (kMaxWorld each) its first tile
// row, its layout-row offset, its padding rows (first, count), and what the
// tile publishes for it (first and last band, head/tail bits and the group
// index); then misc words (layout row of tile row 0, layout rows written,
// the local group's tile rows and first receive row).  The publication
// words are read at the next tile's prologue.
struct DnTabs {
  static constexpr int kLo = 0, kAdd = kMaxWorld, kPad0 = 2 * kMaxWorld, kNpad = 3 * kMaxWorld;
  static constexpr int kB0 = 4 * kMaxWorld, kB1 = 5 * kMaxWorld, kHF = 6 * kMaxWorld;
  static constexpr int kMisc = 7 * kMaxWorld;
  static constexpr int kInts = kMisc + 8;
};
static_assert(kMaxWorld == 64, "one lane of wave 0 per group");

template <class C, bool SWIGLU, bool FLAGS>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::NW / 4, C::NW / 4)))
void grouped_gemm_kernel(PlanLayout L, GemmArgs g, RecvPtrs recv) {
  // one LDS object: the operand rings, and for the down GEMM the epilogue's
  // small tables past them (a second object made the compiler wait for every
  // outstanding load at each K step)
  constexpr int kExtraElems = SWIGLU ? 0 : 2 * (DnTabs::kInts + C::BM);
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_ELEMS + kExtraElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int WAVES_N = C::BN / C::WN;
  const int wave_m = wave / WAVES_N, wave_n = wave % WAVES_N;
  int32_t* hdr = g.ws + L.o_hdr;
  if constexpr (SWIGLU) {
    // the overlapped down GEMM that follows on this stream claims its copy
    // units from these counters
    if (blockIdx.x == 0 && tid == 0) {
      g.sc.claim[0] = 0;
      g.sc.claim[1] = 0;
    }
  }
  const bool overlapped = FLAGS && (int)gridDim.x > g.n_prod;
  if constexpr (FLAGS) {
    // overlapped combine (§5.3): the workgroups past the producers are the
    // consumer.  They are dispatched after every producer of their XCD and
    // hold the GEMM's LDS footprint, so each has a CU of its own; producers
    // never wait for them.
    if ((int)blockIdx.x >= g.n_prod) {
      consume_claimed<C::NT>(L, g.ws, g.sc.claim, g.out, g.flags, g.epoch, recv, g.cc, (int*)lds);
      if (tid == 0) stamp_max(hdr, H_T_CONS_END);
      return;
    }
  }
  if (hdr[H_ERROR] != 0) return;
  // overlapped launch: each producer raises the "started" count (which
  // lets producers that run out of tiles join the consumer once every
  // producer holds its CU) right after its first tile's prologue loads, or
  // when it leaves without a tile.  Raised at the start, the one word's
  // atomics of all producers delayed their first loads (the vector memory
  // counter retires in order): decode-size down GEMMs 44-48 -> 42-46 us.
  bool need_start = overlapped;

  // Row tiles are taken in two regions, each in grouped order: for the down
  // GEMM the remote bands' tiles [0, n_mt_r) before the local bands' (so the
  // tail of the tile order, which the stream-K split finishes last, holds
  // local tiles the consumer does not wait for); gate/up has one region.
  int n_mt, n_nt, n_mt_r;
  if constexpr (SWIGLU) {
    n_mt = hdr[H_GU_MT];
    n_nt = L.gu_ntn;
    n_mt_r = n_mt;
  } else {
    n_mt = hdr[H_DN_MT];
    n_nt = L.dn_ntn;
    n_mt_r = hdr[H_DN_MT_R];
  }
  const int total = n_mt * n_nt;
  const int G = g.n_prod;   // a multiple of 8, at most kMaxProducers
  // Workgroup w runs on XCD w mod 8.  Rounds of G tiles hand each XCD G/8
  // consecutive tiles of the two-level order (operands shared in its L2);
  // a single partial round instead goes round-robin over the XCDs, so that
  // a few tiles do not crowd half the XCDs while the others idle (decode:
  // gate/up 43 -> 35 us, down 34 -> 26 us).
  const int slot = total < G ? (int)blockIdx.x : (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  int blk_r, blk_c;   // the per-XCD block of the tile order
  xcd_block_shape(G >> 3, blk_r, blk_c);
  const int KT = g.K / C::BK;
  const int32_t* rowoff = g.ws + L.o_rowoff;

  // Work split.  The first `full` tiles (whole rounds of G) are taken whole:
  // tile slot, slot + G, ...  When the last round (or the only one, with
  // fewer tiles than workgroups) would be at most 3/4 full and tiles have at
  // least kMinSkKT K steps, its sk_tiles tiles are shared out along K instead
  // ("stream-K"): their
  // sk_tiles * KT K steps are cut into G_sk equal ranges, one per slot below
  // G_sk, each at least kMinSkSteps long.  A range spans at most two tiles;
  // each part (a piece) accumulates its K steps and stores its fp32 partial
  // sums, and the piece that completes a tile's K steps sums all pieces in
  // K order (so the result does not depend on which piece came last) and
  // runs the tile's epilogue.
  int full = total, sk_tiles = 0, G_sk = 0;
  int64_t W_sk = 0;
  if (total > 0 && (KT >= kMinSkKT || (2 * total <= G && KT >= kMinSkKTOneRound))) {
    const int rem = total % G;
    const int64_t w = (int64_t)rem * KT;
    // pieces: at most one per workgroup, at least kMinSkSteps long, and as
    // many as the scratch has slot pairs for (slot 2 * s + piece for
    // s < G_sk); at least one per tile, so that a piece spans at most two
    // tiles
    const int g_sk = (int)min((int64_t)min(G, g.sc.sk_slots / 2), w / kMinSkSteps);
    if (rem != 0 && 4 * rem <= 3 * G && g_sk >= rem) {
      full = total - rem;
      sk_tiles = rem;
      W_sk = w;
      G_sk = g_sk;
    }
  }
  auto sk_lo = [&](int w) { return (int64_t)w * W_sk / G_sk; };
  int64_t sk_cur = 0, sk_hi = 0;
  if (slot < G_sk) {
    sk_cur = sk_lo(slot);
    sk_hi = sk_lo(slot + 1);
  }
  float* sk_part = g.sc.sk_part;
  uint64_t* sk_ctr = g.sc.sk_ctr + (SWIGLU ? 0 : kMaxProducers);

  // load-side lane constants: lane l fills row RPB q + l / CPR, physical chunk
  // l % CPR, so it must fetch the logical chunk swz(row, l % CPR)
  const int ld_row = lane / C::CPR;
  const int ld_phys = lane % C::CPR;
  // read-side lane constants: rows base + (lane & 31) with base a multiple of
  // 32, so the swizzle term depends on the lane only
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int rsw = (lrow / C::R256) % C::CPR;

  // operand rows of this wave inside the LDS tiles
  int prow[C::FN];
#pragma unroll
  for (int i = 0; i < C::FN; ++i) {
    if constexpr (SWIGLU) {
      constexpr int HB = C::BN / 2, HW = C::WN / 2;
      prow[i] = (i < C::FN / 2) ? (wave_n * HW + 32 * i) : (HB + wave_n * HW + 32 * (i - C::FN / 2));
    } else {
      prow[i] = wave_n * C::WN + 32 * i;
    }
  }

  // Down GEMM: a tile is published -- its band heads' and tails' flags set,
  // or counted on their groups' ready words -- once its output stores are
  // acknowledged by every wave.  The wait is not at the end of the tile: the
  // next tile's prologue first issues its loads, then waits for the stores
  // alone (the vector memory counter retires in issue order), so the
  // stores drain under the next tile's loads instead of stalling the waves.
  // The last tile is published after the loop.  What to publish, per group
  // of the tile's expert, is in LDS (DnTabs: written by the epilogue).
  int pend_nt = -1;
  auto publish = [&](int ntile) __attribute__((always_inline)) {
    if (tid >= L.W) return;
    const int* tabs = (const int*)(lds + C::LDS_ELEMS);
    const int b0 = tabs[DnTabs::kB0 + tid];
    if (b0 < 0) return;
    const int b1 = tabs[DnTabs::kB1 + tid], hf = tabs[DnTabs::kHF + tid];
    if (g.cc.signal == 0) {
      // bands b0..b1 of one group: both flags of each, except the first
      // one's head or the last one's tail when they lie in another tile
      for (int b = b0; b <= b1; ++b) {
        uint32_t* f = g.flags + 2 * ((int64_t)b * n_nt + ntile);
        if (b > b0 || (hf & 1)) __hip_atomic_store(f, g.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (b < b1 || (hf & 2)) __hip_atomic_store(f + 1, g.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      // group-batched: the heads and tails counted on the group's
      // epoch-tagged ready word; the group is ready once every band's head
      // and tail have been counted for every column tile
      const uint32_t k = (uint32_t)(2 * (b1 - b0 + 1) - ((hf & 1) ? 0 : 1) - ((hf & 2) ? 0 : 1));
      uint64_t* gready = g.sc.gready + (hf >> 2);
      uint64_t old = __hip_atomic_load(gready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (;;) {
        const uint32_t cnt = ((uint32_t)(old >> 32) == g.epoch ? (uint32_t)old : 0u) + k;
        const uint64_t nv = ((uint64_t)g.epoch << 32) | cnt;
        if (__hip_atomic_compare_exchange_strong(gready, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
          break;
      }
    }
  };
  int t_dp = slot, piece = 0, items = 0;
  for (;;) {
    // next work item: a whole tile, or a piece [kb, ke) of a stream-K tile
    int t, kb = 0, ke = KT, sk_j = -1;
    if (t_dp < full) {
      t = t_dp;
      t_dp += G;
    } else if (sk_cur < sk_hi) {
      sk_j = (int)(sk_cur / KT);
      kb = (int)(sk_cur - (int64_t)sk_j * KT);
      ke = (int)min((int64_t)KT, kb + (sk_hi - sk_cur));
      t = full + sk_j;
      sk_cur += ke - kb;
    } else {
      break;
    }
    ++items;
    int mt, nt;
    if (t < n_mt_r * n_nt) {
      decode_tile<SWIGLU ? kXcdRowsGu : kXcdRowsDn>(t, n_mt_r, n_nt, blk_r, blk_c, mt, nt);
    } else {
      decode_tile<SWIGLU ? kXcdRowsGu : kXcdRowsDn>(t - n_mt_r * n_nt, n_mt - n_mt_r, n_nt, blk_r, blk_c, mt, nt);
      mt += n_mt_r;
    }
    // row tile: up to 256 compacted rows of one expert.  gate/up: row0 the
    // first, row_end the expert's end.  down: its nrows rows of h from crow0
    // on (row0 = 0, row_end = nrows)
    int e, row0, lim, crow0 = 0, nrows = 0;
    if constexpr (SWIGLU) {
      row0 = g.ws[L.o_gumt_row + mt];
      e = g.ws[L.o_gumt_exp + mt];
      lim = g.ws[L.o_crowoff + e + 1];
    } else {
      const ctab_t* tab = (const ctab_t*)g.ws;
      crow0 = tab[L.o_dnt_row + mt];
      e = __builtin_amdgcn_readfirstlane(tab[L.o_dnt_exp + mt]);
      nrows = min(C::BM, tab[L.o_crowoff + e + 1] - crow0);
      row0 = 0;
      lim = nrows;
    }
    // per-tile values are wave-uniform; say so, so that the buffer
    // descriptors built from them live in scalar registers
    e = __builtin_amdgcn_readfirstlane(e);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    crow0 = __builtin_amdgcn_readfirstlane(crow0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    const int row_end = __builtin_amdgcn_readfirstlane(lim);
    const bool empty = row0 >= row_end;
    // A operand.  Every load is bounded by a buffer descriptor, and a lane
    // whose row holds no data gets an offset past the bound (2^31 > the
    // descriptor's extent), where buffer loads return zeros.
    //  * gate/up: row r of the tile is compacted row row0 + r; the table
    //    gives its row of x_recv (gathered) or of the layout X.  Rows of one
    //    tile lie within one X_e, so their layout rows span at most
    //    256 + (W-1)(tb_M-1) rows: 32-bit offsets from the first suffice.
    //  * down: A is h in compacted order: the tile's nrows real rows packed
    //    from crow0 on; its rows past them read zeros.
    __amdgpu_buffer_rsrc_t a_rsrc;
    uint32_t a_off[C::A_LOADS];
    uint32_t b_off[C::B_LOADS];
    if constexpr (SWIGLU) {
      int base = 0;
      if (g.gathered) {
        a_rsrc = make_rsrc(g.a, g.a_bytes);
      } else if (empty) {
        a_rsrc = make_rsrc(g.a, 0);
      } else {
        base = __builtin_amdgcn_readfirstlane(g.rows[row0]);
        const int last = __builtin_amdgcn_readfirstlane(g.rows[min(row0 + C::BM, row_end) - 1]);
        a_rsrc = make_rsrc(g.a + (int64_t)base * g.K, (int64_t)(last - base + 1) * g.K * 2);
      }
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int r = (wave + i * C::NW) * C::RPB + ld_row;
        const int src = (row0 + r < row_end) ? g.rows[row0 + r] - base : -1;
        a_off[i] = src >= 0 ? 2u * ((uint32_t)src * (uint32_t)g.K + (uint32_t)(C::swz(r, ld_phys) * 8))
                            : 0x80000000u;
      }
    } else {
      a_rsrc = make_rsrc(g.a + (int64_t)crow0 * g.K, (int64_t)nrows * g.K * 2);
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        // recomputed per tile (an empty asm hides that it is the same every
        // time): hoisted out of the tile loop these offsets were spilled, and
        // reloading them from scratch would wait for the previous tile's
        // output stores, which the next prologue is meant to overlap
        int r = (wave + i * C::NW) * C::RPB + ld_row;
        asm volatile("" : "+v"(r));
        a_off[i] = r < nrows ? 2u * ((uint32_t)r * (uint32_t)g.K + (uint32_t)(C::swz(r, ld_phys) * 8))
                             : 0x80000000u;
      }
    }
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(g.w + (int64_t)e * g.w_rows * g.K, (int64_t)g.w_rows * g.K * 2);
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      const int r = (wave + i * C::NW) * C::RPB + ld_row;
      int wrow;
      if constexpr (SWIGLU) {
        constexpr int HB = C::BN / 2;
        wrow = (r < HB) ? (nt * HB + r) : (g.half + nt * HB + (r - HB));
      } else {
        wrow = nt * C::BN + r;
      }
      b_off[i] = 2u * ((uint32_t)wrow * (uint32_t)g.K + (uint32_t)(C::swz(r, ld_phys) * 8));
    }

    f32x16 acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int KTt = empty ? 0 : ke - kb;   // K steps of this work item
    // every wave is done with the previous item's LDS stages (and staged
    // output tile) before the prologue below refills them; outstanding
    // output stores are not waited for here
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    __builtin_amdgcn_s_barrier();
    // Stage k of A lives in A buffer k % SA, of B in B buffer k % SB.  Each
    // K step issues the shallow ring's next stage first, then the deep
    // ring's, so at a step's barrier only the deep ring's newest stage may
    // still be in flight.  Prologue: shallow(0), deep(0), then stage 1 of
    // every 3-deep ring.
    auto a_buf = [&](int k) __attribute__((always_inline)) { return (lds_void_t*)(lds + (k % C::SA) * C::A_ELEMS); };
    auto b_buf = [&](int k) __attribute__((always_inline)) { return (lds_void_t*)(lds + C::SA * C::A_ELEMS + (k % C::SB) * C::B_ELEMS); };
    auto issue_a = [&](int k) __attribute__((always_inline)) { issue_operand<C::A_LOADS, C::NW>(a_buf(k), a_rsrc, a_off, (kb + k) * C::BK, wave); };
    auto issue_b = [&](int k) __attribute__((always_inline)) { issue_operand<C::B_LOADS, C::NW>(b_buf(k), b_rsrc, b_off, (kb + k) * C::BK, wave); };
    auto issue_shallow = [&](int k) __attribute__((always_inline)) { if constexpr (C::SA <= C::SB) issue_a(k); else issue_b(k); };
    auto issue_deep = [&](int k) __attribute__((always_inline)) { if constexpr (C::SA <= C::SB) issue_b(k); else issue_a(k); };
    if (KTt > 0) {
      issue_shallow(0);
      issue_deep(0);
    }
    if (KTt > 1) {
      if constexpr (C::SA == 3) issue_a(1);
      if constexpr (C::SB == 3) issue_b(1);
    }
    if (need_start) {
      if (tid == 0) __hip_atomic_fetch_add(g.sc.claim + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      need_start = false;
    }
    if constexpr (FLAGS) {
      if (pend_nt >= 0) {
        // the previous tile's stores went out before the loads just issued:
        // wait for those stores alone, in every wave, then publish the tile
        static_assert(C::A_LOADS + C::B_LOADS <= 63, "vector memory counter range");
        if (KTt > 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(C::A_LOADS + C::B_LOADS));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        __builtin_amdgcn_s_barrier();
        publish(pend_nt);
        pend_nt = -1;
      }
    }

    // One K step.  The barrier waits for stage kt (every later stage but
    // the deep ring's newest has been issued after it) and retires every LDS
    // read of the buffers refilled next.  Operand fragments run one 16-wide
    // k-substep ahead of the MFMAs (two register sets), so at most
    // 2 (FN + FM) LDS reads are outstanding and each substep waits only for
    // its own fragments; the next stages' global->LDS loads go out after the
    // first substep's reads.  Steady-state steps issue both rings, the last
    // S_DEEP-1 steps fewer, so each step body is one branch-free scheduling
    // region.  FE (<= FM) is the number of this wave's 32-row blocks that
    // take part: blocks past it hold padding rows only, and their
    // accumulators stay zero.
    auto k_step = [&](int kt, auto issue_sh_tag, auto issue_dp_tag, int in_flight, auto fe_tag)
                      __attribute__((always_inline)) {
      constexpr bool ISSUE_SH = decltype(issue_sh_tag)::value;
      constexpr bool ISSUE_DP = decltype(issue_dp_tag)::value;
      constexpr int FE = decltype(fe_tag)::value;
      constexpr int FNE = FE > 0 ? C::FN : 0;
      stage_barrier<C>(in_flight);
      const uint16_t* sa = lds + (kt % C::SA) * C::A_ELEMS;
      const uint16_t* sb = lds + C::SA * C::A_ELEMS + (kt % C::SB) * C::B_ELEMS;
      bf16x8 pw[2][C::FN], px[2][C::FM];
      auto read_frags = [&](int kk, int slot) __attribute__((always_inline)) {
        const int phys = ((2 * kk + lhalf) ^ rsw) * 8;
#pragma unroll
        for (int i = 0; i < FNE; ++i)
          pw[slot][i] = *(const bf16x8*)(sb + (prow[i] + lrow) * C::BK + phys);
#pragma unroll
        for (int j = 0; j < FE; ++j)
          px[slot][j] = *(const bf16x8*)(sa + (wave_m * C::WM + 32 * j + lrow) * C::BK + phys);
      };
      read_frags(0, 0);
      if constexpr (ISSUE_SH) issue_shallow(kt + C::S_SHALLOW - 1);
      if constexpr (ISSUE_DP) issue_deep(kt + C::S_DEEP - 1);
      // gate/up: this wave's MFMA block at raised wave priority, so the other
      // wave of the SIMD does not delay it (Mixtral-like gate/up 1758 ->
      // 1745 us; the down GEMM got 4-5% slower with it, so only here)
      if constexpr (SWIGLU) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        if (kk + 1 < C::KK) read_frags(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int i = 0; i < FNE; ++i)
#pragma unroll
          for (int j = 0; j < FE; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pw[kk & 1][i], px[kk & 1][j], acc[i][j], 0, 0, 0);
      }
      if constexpr (SWIGLU) __builtin_amdgcn_s_setprio(0);
      constexpr int NVMEM = (ISSUE_SH ? (C::SA <= C::SB ? C::A_LOADS : C::B_LOADS) : 0) +
                            (ISSUE_DP ? (C::SA <= C::SB ? C::B_LOADS : C::A_LOADS) : 0);
      if constexpr (FE > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, FNE + FE, 0);
      if constexpr (NVMEM > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmem, NVMEM, 0);
      if constexpr (FE > 0) {
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
          if (kk + 1 < C::KK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, FNE + FE, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, FNE * FE, 0);
        }
      }
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    // one loop per step body (a branch between bodies inside one loop makes
    // the register allocator spill)
    auto run_k = [&](auto fe_tag) __attribute__((always_inline)) {
      int kt = 0;
      for (; kt + C::S_DEEP - 1 < KTt; ++kt) k_step(kt, T_{}, T_{}, C::DEEP_LOADS, fe_tag);
      if constexpr (C::S_DEEP > C::S_SHALLOW)
        for (; kt + C::S_SHALLOW - 1 < KTt; ++kt) k_step(kt, T_{}, F_{}, (kt + 1 < KTt) ? C::DEEP_LOADS : 0, fe_tag);
      for (; kt < KTt; ++kt) k_step(kt, F_{}, F_{}, (kt + 1 < KTt) ? C::DEEP_LOADS : 0, fe_tag);
    };
    if constexpr (!SWIGLU) {
      // The tile's nrows real rows are packed at its top.  This wave's
      // blocks are rows [wave_m WM + 32 j, +32), j < FM; it multiplies
      // blocks 0 .. fe - 1, the last of them holding a real row, and every
      // wave still joins every load and barrier.  The waves of one SIMD hold
      // the two row halves of the same columns, so the SIMD's MFMA time
      // follows the tile's real rows.
      int fe = (nrows + 31) / 32 - wave_m * C::FM;
      fe = __builtin_amdgcn_readfirstlane(max(0, min(C::FM, fe)));
      static_assert(C::FM == 4, "one K-loop body per block count");
      switch (fe) {
        case 4: run_k(std::integral_constant<int, 4>{}); break;
        case 3: run_k(std::integral_constant<int, 3>{}); break;
        case 2: run_k(std::integral_constant<int, 2>{}); break;
        case 1: run_k(std::integral_constant<int, 1>{}); break;
        default: run_k(std::integral_constant<int, 0>{}); break;
      }
    } else {
      // gate/up: the same over the tile's compacted rows (the last tile of
      // an expert is partial).  A SIMD holds waves wave_m and wave_m + 2, so
      // a tile of at most 128 rows halves the busiest SIMD's MFMA time.
      const int rows_t = min(C::BM, row_end - row0);
      int fe = (rows_t + 31) / 32 - wave_m * C::FM;
      fe = __builtin_amdgcn_readfirstlane(max(0, min(C::FM, fe)));
      static_assert(C::FM == 2, "one K-loop body per block count");
      switch (fe) {
        case 2: run_k(std::integral_constant<int, 2>{}); break;
        case 1: run_k(std::integral_constant<int, 1>{}); break;
        default: run_k(std::integral_constant<int, 0>{}); break;
      }
    }

    if (sk_j >= 0) {
      // stream-K piece: store the partial sums in register order (slot
      // 2*slot + piece, [float4 c][thread]), publish them, count this piece's
      // K steps on the tile's epoch-tagged counter; the piece that completes
      // KT adds every other piece's partials and goes on to the epilogue.
      // Published like the down GEMM's tiles: device-scope (sc1) stores,
      // acknowledged by every wave before the counter update, and read back
      // with sc1 loads, so no L2 write-back is needed.
      const __amdgpu_buffer_rsrc_t mine =
          make_rsrc(sk_part + (int64_t)(2 * slot + piece) * C::BM * C::BN, (int64_t)C::BM * C::BN * 4);
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v4u32 pv;
#pragma unroll
            for (int c = 0; c < 4; ++c) pv[c] = __float_as_uint(acc[i][j][4 * q + c]);
            __builtin_amdgcn_raw_buffer_store_b128(pv, mine, (((i * C::FM + j) * 4 + q) * C::NT + tid) * 16, 0,
                                                   kDeviceScope);
          }
      wait_vm0();
      __syncthreads();   // also: every wave is done with the LDS ring
      int* s_last = (int*)lds;
      if (tid == 0) {
        uint64_t* ctr = sk_ctr + sk_j;
        uint64_t old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t cnt;
        for (;;) {
          cnt = ((uint32_t)(old >> 32) == g.epoch ? (uint32_t)old : 0u) + (uint32_t)(ke - kb);
          const uint64_t nv = ((uint64_t)g.epoch << 32) | cnt;
          if (__hip_atomic_compare_exchange_strong(ctr, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT))
            break;
        }
        *s_last = (cnt == (uint32_t)KT);
      }
      __syncthreads();
      const int last = *s_last;
      ++piece;
      if (!last) continue;
      // the tile's K range [sk_j*KT, (sk_j+1)*KT) meets the ranges of slots
      // w_a..w_b (ascending K); each holds it as its first (piece 0) or
      // second piece.  Sum all of them in that order -- this slot's own
      // partial re-read from memory like the others -- so the result does
      // not depend on which piece came last.  Pieces outside, and for each
      // piece half the tile's loads in flight at once: the loads bypass this
      // XCD's caches and their latency, not their bytes, sets the cost.
      const int64_t a0 = (int64_t)sk_j * KT, a1 = a0 + KT;
      int wa = (int)(a0 * G_sk / W_sk);
      while (wa > 0 && sk_lo(wa) > a0) --wa;
      while (wa + 1 < G_sk && sk_lo(wa + 1) <= a0) ++wa;
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      constexpr int FH = (C::FN + 1) / 2;   // blocks of i per half
      for (int w = wa; w < G_sk && sk_lo(w) < a1; ++w) {
        const int pw_idx = (sk_lo(w) / KT == sk_j) ? 0 : 1;
        // 16-byte agent-scope (sc1) loads: the partial may come from another
        // XCD, so this XCD's cached lines of the slot must not be used
        const __amdgpu_buffer_rsrc_t prs =
            make_rsrc(sk_part + (int64_t)(2 * w + pw_idx) * C::BM * C::BN, (int64_t)C::BM * C::BN * 4);
#pragma unroll
        for (int h = 0; h < C::FN; h += FH) {
          v4u32 ld[FH][C::FM][4];
#pragma unroll
          for (int i = 0; i < FH; ++i)
#pragma unroll
            for (int j = 0; j < C::FM; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                if (h + i < C::FN)
                  ld[i][j][q] = __builtin_amdgcn_raw_buffer_load_b128(
                      prs, (((h + i) * C::FM + j) * 4 + q) * C::NT * 16 + tid * 16, 0, kDeviceScope);
              }
#pragma unroll
          for (int i = 0; i < FH; ++i)
#pragma unroll
            for (int j = 0; j < C::FM; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                if (h + i < C::FN) {
#pragma unroll
                  for (int c = 0; c < 4; ++c) acc[h + i][j][4 * q + c] += __uint_as_float(ld[i][j][q][c]);
                }
              }
        }
      }
    }

    // Epilogue.  A lane holds rows wave_m*WM + 32j + (lane & 31) and, per
    // (i, q), 4 consecutive columns 32i + 8q + 4*(lane/32) of its wave's
    // block.
    if constexpr (SWIGLU) {
      // gate/up: h = silu(gate) * up straight from registers, 8 bytes per
      // lane (staging this 256 x 128 tile through LDS measured 1-4% slower,
      // and pairing lanes l, l+32 with v_permlane32_swap into 16-byte
      // stores 0.4-1.8% slower)
      constexpr int HB = C::BN / 2, HW = C::WN / 2;
      const int mrow0 = row0 + wave_m * C::WM + lrow;
      const int ncol0 = nt * HB + wave_n * HW + 4 * lhalf;
#pragma unroll
      for (int j = 0; j < C::FM; ++j) {
        const int m = mrow0 + 32 * j;
        if (m < row_end) {
          uint16_t* orow = g.out + (int64_t)m * g.out_cols;
#pragma unroll
          for (int i = 0; i < C::FN / 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float hv[4];
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const float gt = acc[i][j][4 * q + v];
                const float up = acc[i + C::FN / 2][j][4 * q + v];
                hv[v] = silu_f(gt) * up;
              }
              uint2 pk;
              pk.x = pack_bf16x2(hv[0], hv[1]);
              pk.y = pack_bf16x2(hv[2], hv[3]);
              *(uint2*)(orow + ncol0 + 32 * i + 8 * q) = pk;
            }
        }
      }
      wait_vm0();
    } else {
      // Down GEMM: stored straight from registers, each store instruction
      // would touch 32 rows with 8 bytes per lane, i.e. 16-byte pieces of 32
      // cache lines, and every one of them must be acknowledged before the
      // tile's release.  The tile goes through LDS instead (the ring is idle
      // now): every lane writes its bf16 values there, then each thread
      // stores 16-byte chunks of whole output rows, so a wavefront writes
      // whole lines.  LDS layout: row-major, BN bf16 per row, the 16-byte
      // chunk c of row m at c ^ (m mod NCH), so that 16 lanes reading 16
      // consecutive chunks of one row touch 16 distinct bank groups.
      constexpr int OUT_TC = C::BN;     // output columns of the tile
      constexpr int NCH = OUT_TC / 8;   // 16-byte chunks per output row
      static_assert(C::BM * OUT_TC <= C::LDS_ELEMS, "output tile fits the LDS ring");
      static_assert((NCH & (NCH - 1)) == 0 && NCH >= 16, "power-of-two chunk count");
      // The tile's rows run through the groups of X_e in layout order
      // (remote owners ascending, r skipped, then r), each group's rows
      // consecutive in both h and the layout (a remote group's padding rows
      // follow its last real row).  Lane k < W of wave 0 takes group k: the
      // tile rows [lo, hi) it holds, the layout row of each (tile row m ->
      // m + add, counted from the layout row of tile row 0), the padding
      // rows to zero when the tile holds the end of a remote group, and the
      // bands to publish -- with whether the first one's head and the last
      // one's tail lie in this tile.  A lane past W, or a group with no row
      // here, has lo = hi (and b0 = -1), so tile row m belongs to the last
      // group k < W with lo <= m.
      int* tabs = (int*)(lds + C::LDS_ELEMS);
      int* rowmap = tabs + DnTabs::kInts;   // [BM] layout row of each tile row (relative), or -1
      int k_o = 0, k_n = 0, k_gc = 0, k_grow = 0, k_band = 0, k_base = 0;
      const bool k_on = tid < L.W;
      if (k_on) {
        k_o = tid < L.W - 1 ? (tid < L.r ? tid : tid + 1) : L.r;
        const int gi = e * L.W + k_o;
        k_n = g.ws[L.o_c + gi];
        k_gc = g.ws[L.o_gcrow + gi] - crow0;   // the group's first row, relative to the tile
        k_grow = g.ws[L.o_grow + gi];
        k_band = g.ws[L.o_gband + gi];
        if (k_o == L.r) k_base = g.ws[L.o_base + L.r * L.E_l + e];
      }
      __syncthreads();   // every wave is done with the ring
      char* tl = (char*)lds;
#pragma unroll
      for (int j = 0; j < C::FM; ++j) {
        const int m = wave_m * C::WM + 32 * j + lrow;
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 pk;
            pk.x = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
            pk.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            const int ch = wave_n * (C::WN / 8) + 4 * i + q;
            *(uint2*)(tl + m * (OUT_TC * 2) + 16 * (ch ^ (m & (NCH - 1))) + 8 * lhalf) = pk;
          }
      }
      if (tid < 64) {
        const int lo = k_on ? min(max(k_gc, 0), nrows) : nrows;
        const int hi = k_on ? min(max(k_gc + k_n, 0), nrows) : nrows;
        // tile row 0 lies in exactly one group (nrows >= 1)
        const uint64_t at0 = __ballot(k_on && lo == 0 && hi > 0);
        const int lbase = __shfl(k_grow - k_gc, (int)__builtin_ctzll(at0));
        const int add = k_grow - k_gc - lbase;
        const bool ends = hi > lo && k_gc + k_n <= nrows;   // the group's last row is in the tile
        const int npad = (ends && k_o != L.r) ? fdiv(k_n + L.tb_m - 1, L.div_tb) * L.tb_m - k_n : 0;
        int end_rel = hi > lo ? hi + add + npad : 0;   // layout rows written, from tile row 0's
#pragma unroll
        for (int xs = 1; xs < 64; xs <<= 1) end_rel = max(end_rel, __shfl_xor(end_rel, xs));
        int b0 = -1, b1 = -1, hf = 0;
        if (hi > lo) {
          const int q0 = fdiv(lo - k_gc, L.div_tb), q1 = fdiv(hi - 1 - k_gc, L.div_tb);
          b0 = k_band + q0;
          b1 = k_band + q1;
          const bool head0 = lo - k_gc == q0 * L.tb_m;
          const bool tail1 = hi - k_gc == min((q1 + 1) * L.tb_m, k_n);
          hf = (head0 ? 1 : 0) | (tail1 ? 2 : 0) | ((e * L.W + k_o) << 2);
        }
        tabs[DnTabs::kLo + tid] = lo;
        tabs[DnTabs::kAdd + tid] = add;
        tabs[DnTabs::kPad0 + tid] = npad > 0 ? hi + add : 0;
        tabs[DnTabs::kNpad + tid] = npad;
        tabs[DnTabs::kB0 + tid] = b0;
        tabs[DnTabs::kB1 + tid] = b1;
        tabs[DnTabs::kHF + tid] = hf;
        if (tid == 0) {
          tabs[DnTabs::kMisc + 0] = lbase;
          tabs[DnTabs::kMisc + 1] = end_rel;
        }
        if (k_on && k_o == L.r) {
          tabs[DnTabs::kMisc + 2] = lo;
          tabs[DnTabs::kMisc + 3] = hi;
          tabs[DnTabs::kMisc + 4] = k_base + (lo - k_gc);   // receive row of the first local row here
        }
      }
      __syncthreads();
      if (tid < C::BM) {
        const int m = tid;
        int dst = -1;
        if (m < nrows) {
          int lo = 0, hi = L.W - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tabs[DnTabs::kLo + mid] <= m) lo = mid; else hi = mid - 1;
          }
          dst = m + tabs[DnTabs::kAdd + lo];
        }
        rowmap[m] = dst;
      }
      __syncthreads();
      // the stores: the tile's real rows to their layout rows (and its rows
      // of the local group also to the rank's own receive buffer), then
      // zeros into the padding rows of every remote group that ends here;
      // the descriptors end past the last row written
      const int64_t out_row_bytes = (int64_t)g.out_cols * 2;
      const int col0 = nt * OUT_TC;
      const int lbase = __builtin_amdgcn_readfirstlane(tabs[DnTabs::kMisc + 0]);
      const int span = __builtin_amdgcn_readfirstlane(tabs[DnTabs::kMisc + 1]);
      // the local group's rows here and the receive row of the first (the
      // local group's lane writes them for every tile; lo = hi if none)
      const int llo = __builtin_amdgcn_readfirstlane(tabs[DnTabs::kMisc + 2]);
      const int lhi = __builtin_amdgcn_readfirstlane(tabs[DnTabs::kMisc + 3]);
      const int lrecv = __builtin_amdgcn_readfirstlane(tabs[DnTabs::kMisc + 4]);
      if (nrows > 0) {
        const __amdgpu_buffer_rsrc_t o_rsrc =
            make_rsrc(g.out + (int64_t)lbase * g.out_cols + col0, (int64_t)span * out_row_bytes);
        const bool has_local = lhi > llo;
        __amdgpu_buffer_rsrc_t l_rsrc = o_rsrc;
        if (has_local)
          l_rsrc = make_rsrc(recv.p[L.r] + (int64_t)lrecv * g.out_cols + col0, (int64_t)(lhi - llo) * out_row_bytes);
        constexpr int RPP = C::NT / NCH;   // rows per pass
        constexpr int PASSES = C::BM / RPP;
        constexpr int UNR = PASSES >= 4 ? 4 : PASSES;
        static_assert(PASSES % UNR == 0, "whole unrolled passes");
        const int ch = tid % NCH;
        const int r_in = tid / NCH;
        for (int p0 = 0; p0 < PASSES; p0 += UNR) {
          if ((p0 * RPP) >= nrows) break;
          v4u32 v[UNR];
          int dst[UNR];
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            const int m = (p0 + u) * RPP + r_in;
            v[u] = *(const v4u32*)(tl + m * (OUT_TC * 2) + 16 * (ch ^ (m & (NCH - 1))));
            dst[u] = rowmap[m];
          }
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            const int m = (p0 + u) * RPP + r_in;
            const uint32_t off = dst[u] >= 0 ? (uint32_t)((int64_t)dst[u] * out_row_bytes + ch * 16) : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b128(v[u], o_rsrc, off, 0, MOE_STORE_AUX);
            if (has_local) {
              const uint32_t loff =
                  (m >= llo && m < lhi) ? (uint32_t)((int64_t)(m - llo) * out_row_bytes + ch * 16) : 0xFFFFFFF0u;
              __builtin_amdgcn_raw_buffer_store_b128(v[u], l_rsrc, loff, 0, MOE_STORE_AUX);
            }
          }
        }
        // padding rows of the remote groups that end in this tile
        const v4u32 z = {0u, 0u, 0u, 0u};
        for (int k = 0; k < L.W; ++k) {
          const int npad = tabs[DnTabs::kNpad + k];
          if (npad == 0) continue;
          const int pad0 = tabs[DnTabs::kPad0 + k];
          for (int idx = tid; idx < npad * NCH; idx += C::NT) {
            const int row = pad0 + idx / NCH;
            __builtin_amdgcn_raw_buffer_store_b128(z, o_rsrc, (uint32_t)((int64_t)row * out_row_bytes + (idx % NCH) * 16),
                                                   0, MOE_STORE_AUX);
          }
        }
      }
      // Publication.  Every row this tile hands to the consumer was stored
      // at device scope (sc1: written through this XCD's L2 to the memory
      // side, the point where all XCDs' agent-scope loads meet; the same
      // instruction form as a relaxed agent-scope atomic store), and each
      // wave waits until its stores are acknowledged (at the next tile's
      // prologue, see `publish`); after a barrier the flags are set with
      // relaxed agent-scope stores.  So the data is
      // visible to every XCD before any flag is, without the L2 write-back an
      // agent-scope release fence would add: that write-back (buffer_wbl2)
      // only matters for ordinary write-back stores, and walking the L2 once
      // per tile cost 7-10% of the short-K down GEMMs.  The consumer polls
      // the flags with relaxed agent-scope loads and reads the rows only
      // after it has seen them (a control dependency), with agent-scope (sc1)
      // loads that do not return lines this XCD cached earlier; it issues no
      // acquire fence and no L2 invalidate.
      static_assert((MOE_STORE_AUX & kDeviceScope) != 0, "flag publication needs device-scope (sc1) output stores");
      if constexpr (FLAGS) {
        pend_nt = nt;   // published once the stores above are acknowledged
      } else {
        wait_vm0();
      }
    }
  }
  if constexpr (FLAGS) {
    if (pend_nt >= 0) {   // the last tile: its stores are the last memory operations
      wait_vm0();
      __builtin_amdgcn_s_barrier();
      publish(pend_nt);
    }
    if (need_start && tid == 0) __hip_atomic_fetch_add(g.sc.claim + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) stamp_max(hdr, H_T_PROD_END);
    if (overlapped && items > 0) {
      // out of tiles: help copy the remaining remote segments, but only once
      // every producer has started -- a producer still waiting for a CU could
      // otherwise be kept from it by workgroups that wait for its tiles.
      // A producer that got no tile at all (a grid larger than the tile
      // count) leaves instead: joining at once, it would only poll flags
      // beside the producers still computing (measured on a decode-size
      // layer: 5 us slower down GEMM).
      __syncthreads();   // every wave is done with the LDS ring
      int* s_word = (int*)lds;
      if (tid == 0) s_word[0] = __hip_atomic_load(g.sc.claim + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const bool all_started = s_word[0] == g.n_prod;
      __syncthreads();
      if (all_started) {
        consume_claimed<C::NT>(L, g.ws, g.sc.claim, g.out, g.flags, g.epoch, recv, g.cc, s_word);
        if (tid == 0) stamp_max(hdr, H_T_CONS_END);
      }
    }
  }
}


using GuCfg = Cfg<256, 256, MOE_GU_WAVES_M, MOE_GU_WAVES_N, MOE_GU_BK, MOE_GU_SA, MOE_GU_SB>;
static_assert(GuCfg::BK == kGuBK, "the host sizes the stream-K scratch with this K step");
using Dn256 = Cfg<256, 256, MOE_DN_WAVES_M, MOE_DN_WAVES_N, MOE_DN_BK, MOE_DN_SA, MOE_DN_SB>;
static_assert(Dn256::BK == kDnBK, "the host sizes the stream-K scratch with this K step");
static_assert(Dn256::BM == kDnBM, "the planner cuts the down tiles at this height");

__global__ __launch_bounds__(256) void clear_counters_kernel(Scratch sc) {
  for (int i = threadIdx.x; i < 2 * kMaxProducers; i += blockDim.x) sc.sk_ctr[i] = 0;
  for (int i = threadIdx.x; i < kMaxWorld; i += blockDim.x) sc.link_free[i] = 0;
  for (int i = threadIdx.x; i < kMaxGroups; i += blockDim.x) sc.gready[i] = 0;
  if (threadIdx.x < 2) sc.claim[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_clear_counters(const Scratch& sc, hipStream_t s) {
  hipLaunchKernelGGL(clear_counters_kernel, dim3(1), dim3(256), 0, s, sc);
  return hipGetLastError();
}

hipError_t launch_gateup(const PlanLayout& L, int32_t* ws, const Scratch& sc, const uint16_t* x, bool gathered,
                         const uint16_t* wgu, uint16_t* h, uint32_t epoch, int grid, hipStream_t s) {
  GemmArgs a{ws, x, wgu, h, nullptr, epoch, L.d, L.f, 2 * L.f, L.f, grid, CopyCtl{},
             ws + (gathered ? L.o_cmpsrc : L.o_cmprow), gathered ? 1 : 0, gathered ? (int64_t)L.R * L.d * 2 : 0, sc};
  RecvPtrs none{};
  hipLaunchKernelGGL((grouped_gemm_kernel<GuCfg, true, false>), dim3(grid), dim3(GuCfg::NT), 0, s, L, a, none);
  return hipGetLastError();
}

hipError_t launch_down(const PlanLayout& L, int32_t* ws, const Scratch& sc, const uint16_t* h, const uint16_t* wd,
                       uint16_t* y, uint32_t* flags, uint32_t epoch, const RecvPtrs& recv, const CopyCtl& cc,
                       int n_prod, int grid, hipStream_t s) {
  GemmArgs a{ws, h, wd, y, flags, epoch, L.f, L.d, L.d, 0, n_prod, cc, nullptr, 0, 0, sc};
  hipLaunchKernelGGL((grouped_gemm_kernel<Dn256, false, true>), dim3(grid), dim3(Dn256::NT), 0, s, L, a, recv);
  return hipGetLastError();
}

}  // namespace moe
