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
//     4 wavefronts per workgroup, each owning a WM x WN register tile.
//   * The MFMA's first operand is the weight tile (rows = output columns n),
//     the second the activation tile (rows = output rows m), so each lane ends
//     with 4 consecutive output columns per accumulator quad: 8-byte bf16
//     stores, and the SwiGLU gate/up pair of a column sits in one lane.
//   * K steps of 64: both operands are K-contiguous in HBM, copied straight
//     into LDS with 16-byte global_load_lds (no staging registers), two LDS
//     stages, 16-byte chunks XOR-swizzled by (row mod 8) so that the
//     ds_read_b128 operand fetches are bank-conflict free.
//   * Persistent grid (a multiple of 8 workgroups).  Workgroup w runs on XCD
//     w mod 8; it takes slot (w mod 8) * (G/8) + w/8 of every round of G
//     tiles, so each XCD works on a contiguous run of the tile order, and the
//     tile order groups GM row tiles per column sweep so the run shares
//     operand rows in that XCD's L2.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Tile shapes (compile-time; the defaults are the measured best on MI355X).
#ifndef MOE_GROUP_M
#define MOE_GROUP_M 8
#endif
#ifndef MOE_GU_WAVES_M
#define MOE_GU_WAVES_M 4
#endif
#ifndef MOE_GU_WAVES_N
#define MOE_GU_WAVES_N 2
#endif
#ifndef MOE_DN_WAVES_M
#define MOE_DN_WAVES_M 4
#endif
#ifndef MOE_DN_WAVES_N
#define MOE_DN_WAVES_N 2
#endif
#ifndef MOE_BK
#define MOE_BK 64
#endif
#ifndef MOE_STAGES
#define MOE_STAGES 2
#endif
constexpr int kGroupM = MOE_GROUP_M;   // row tiles per column sweep

// BM x BN output tile, WAVES_M x WAVES_N wavefronts, K step BK, STAGES-deep
// global -> LDS ring.  An LDS row holds BK bf16 (BK/8 chunks of 16 bytes);
// chunks are XOR-swizzled so that any 16 lanes reading 16 consecutive rows at
// the same logical chunk touch 16 distinct 16-byte bank groups of gfx950's
// 64-bank LDS (one ds_read_b128 phase).
template <int BM_, int BN_, int WAVES_M, int WAVES_N, int BK_, int STAGES_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
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
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = STAGES * STAGE_ELEMS * 2;
  static constexpr int A_LOADS = BM / RPB / NW;  // 1 KB wave loads per stage and wave
  static constexpr int B_LOADS = BN / RPB / NW;
  static constexpr int LPW = A_LOADS + B_LOADS;
  static_assert(NW == 4 || NW == 8, "four or eight wavefronts per workgroup");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "every wavefront loads both operands");
  static_assert(BM % (RPB * NW) == 0 && BN % (RPB * NW) == 0, "whole wave loads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  static_assert(LPW * (STAGES - 2) <= 63, "vmcnt range");
  __device__ static int swz(int row, int c) { return c ^ ((row / R256) % CPR); }
};

struct GemmArgs {
  const int32_t* ws;
  const uint16_t* a;      // activations [rows, K]
  const uint16_t* w;      // weights [E_l, N_total, K]
  uint16_t* out;          // [rows, out_cols]
  uint32_t* flags;
  uint32_t epoch;
  int K;                  // reduction length
  int out_cols;           // columns of `out`
  int w_rows;             // rows of one expert's weight matrix
  int half;               // SWIGLU: f (offset of the up rows); else 0
};

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for the K loop: this wavefront waits until at most
// `stages_in_flight` later stages of its own global->LDS loads are
// outstanding (so the current stage has landed) and its LDS reads are done,
// then all wavefronts meet.  __syncthreads() would also wait for every
// outstanding load (vmcnt(0)) and so drain the prefetch ring.
template <int LPW>
__device__ __forceinline__ void stage_barrier(int stages_in_flight) {
  switch (stages_in_flight) {
    case 0: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LPW) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LPW) : "memory"); break;
  }
}

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x8, kSchedVmem = 0x10, kSchedDsRead = 0x100;

// Tile t of a (n_mt x n_nt) grid in grouped order -> (mt, nt): groups of
// kGroupM row tiles sweep all column tiles.
__device__ __forceinline__ void decode_tile(int t, int n_mt, int n_nt, int& mt, int& nt) {
  const int per_group = kGroupM * n_nt;
  const int g = t / per_group;
  const int in = t - g * per_group;
  const int gm = min(kGroupM, n_mt - g * kGroupM);
  mt = g * kGroupM + in % gm;
  nt = in / gm;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ float silu_f(float g) {
  // silu(g) = g / (1 + e^-g), e^-g = 2^(-g log2 e)
  return g / (1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

template <class C>
__device__ __forceinline__ void issue_stage(lds_void_t* lds_stage, const char* a_base, const uint32_t (&a_off)[C::A_LOADS],
                                            const char* b_base, const uint32_t (&b_off)[C::B_LOADS], int k0,
                                            int wave) {
  // wave `wave` fills LDS rows [RPB q, RPB (q+1)) for q = wave, wave + NW, ...;
  // the lane byte offsets (from wave-uniform bases) carry the swizzled chunk
  char* base = (char*)lds_stage;
  const char* a = a_base + 2 * k0;
  const char* b = b_base + 2 * k0;
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int q = wave + i * C::NW;
    __builtin_amdgcn_global_load_lds((const void*)(a + a_off[i]), (lds_void_t*)(base + q * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int q = wave + i * C::NW;
    __builtin_amdgcn_global_load_lds((const void*)(b + b_off[i]), (lds_void_t*)(base + C::A_ELEMS * 2 + q * 1024),
                                     16, 0, 0);
  }
}

template <class C, bool SWIGLU, bool FLAGS>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::NW / 4, C::NW / 4)))
void grouped_gemm_kernel(PlanLayout L, GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::STAGES * C::STAGE_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int WAVES_N = C::BN / C::WN;
  const int wave_m = wave / WAVES_N, wave_n = wave % WAVES_N;
  const int32_t* hdr = g.ws + L.o_hdr;
  if (hdr[H_ERROR] != 0) return;

  int n_mt, n_nt;
  if constexpr (SWIGLU) {
    n_mt = hdr[H_GU_MT];
    n_nt = L.gu_ntn;
  } else {
    n_mt = hdr[H_BANDS] * L.dn_sub;
    n_nt = L.dn_ntn;
  }
  const int total = n_mt * n_nt;
  const int G = gridDim.x;
  const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int KT = g.K / C::BK;
  const int32_t* rowoff = g.ws + L.o_rowoff;

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

  for (int t = slot; t < total; t += G) {
    int mt, nt;
    decode_tile(t, n_mt, n_nt, mt, nt);
    int e, row0;
    if constexpr (SWIGLU) {
      row0 = g.ws[L.o_gumt_row + mt];
      e = g.ws[L.o_gumt_exp + mt];
    } else {
      const int band = mt / L.dn_sub;
      e = g.ws[L.o_bexp + band];
      row0 = g.ws[L.o_bsrc + band] + (mt - band * L.dn_sub) * C::BM;
    }
    const int row_end = rowoff[e + 1];
    // a sub-tile of a partial (local tail) band can start past the expert's
    // last row: nothing to compute or store, only its flag to publish
    const bool empty = row0 >= row_end;
    // wave-uniform base row (clamped into the expert) + 32-bit lane byte
    // offsets, never negative (rows < 2^16 apart, K < 2^16)
    const int rbase = min(row0, row_end - 1);
    const char* a_base = (const char*)(g.a + (int64_t)rbase * g.K);
    const char* b_base = (const char*)(g.w + (int64_t)e * g.w_rows * g.K);
    uint32_t a_off[C::A_LOADS];
    uint32_t b_off[C::B_LOADS];
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int r = (wave + i * C::NW) * C::RPB + ld_row;
      const int rr = min(row0 + r, row_end - 1) - rbase;
      a_off[i] = 2u * ((uint32_t)rr * (uint32_t)g.K + (uint32_t)(C::swz(r, ld_phys) * 8));
    }
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

    const int KTt = empty ? 0 : KT;   // K steps of this tile
    // every wave is done with the previous tile's LDS stages before the
    // prologue below refills them
    __syncthreads();
    // prologue: the first STAGES-1 stages in flight
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s)
      if (s < KTt)
        issue_stage<C>((lds_void_t*)(lds + s * C::STAGE_ELEMS), a_base, a_off, b_base, b_off, s * C::BK, wave);

    for (int kt = 0; kt < KTt; ++kt) {
      // stage kt has landed once at most min(STAGES-2, KT-1-kt) later stages
      // of this wave are still in flight; the barrier makes it true for all
      // waves and also retires every read of the buffer refilled next
      stage_barrier<C::LPW>(min(C::STAGES - 2, KT - 1 - kt));
      const uint16_t* sa = lds + (kt % C::STAGES) * C::STAGE_ELEMS;
      const uint16_t* sb = sa + C::A_ELEMS;
      // all fragments of the stage first, the next stage's loads in between,
      // then the MFMAs (the first ones wait only for the first fragments)
      bf16x8 pw[C::KK][C::FN], px[C::KK][C::FM];
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        const int phys = ((2 * kk + lhalf) ^ rsw) * 8;
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
          pw[kk][i] = *(const bf16x8*)(sb + (prow[i] + lrow) * C::BK + phys);
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
          px[kk][j] = *(const bf16x8*)(sa + (wave_m * C::WM + 32 * j + lrow) * C::BK + phys);
        if (kk == 0 && kt + C::STAGES - 1 < KT)
          issue_stage<C>((lds_void_t*)(lds + ((kt + C::STAGES - 1) % C::STAGES) * C::STAGE_ELEMS), a_base, a_off,
                         b_base, b_off, (kt + C::STAGES - 1) * C::BK, wave);
      }
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
          for (int j = 0; j < C::FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pw[kk][i], px[kk][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::FN + C::FM, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmem, C::LPW, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, (C::KK - 1) * (C::FN + C::FM), 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, C::KK * C::FN * C::FM, 0);
    }

    // epilogue: lane holds rows m = .. + (lane & 31), columns n = .. + 8*(v/4) + 4*(lane/32) + v%4
    const int mrow0 = row0 + wave_m * C::WM + lrow;
    if constexpr (SWIGLU) {
      constexpr int HB = C::BN / 2, HW = C::WN / 2;
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
      const int ncol0 = nt * C::BN + wave_n * C::WN + 4 * lhalf;
#pragma unroll
      for (int j = 0; j < C::FM; ++j) {
        const int m = mrow0 + 32 * j;
        if (m < row_end) {
          uint16_t* orow = g.out + (int64_t)m * g.out_cols;
#pragma unroll
          for (int i = 0; i < C::FN; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint2 pk;
              pk.x = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
              pk.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
              *(uint2*)(orow + ncol0 + 32 * i + 8 * q) = pk;
            }
        }
      }
      // every wave's stores have reached L2; then one release at agent scope
      // (L2 write-back) before the flag of this tile is set
      wait_vm0();
      if constexpr (FLAGS) {
        __syncthreads();
        if (tid == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          __hip_atomic_store(g.flags + (int64_t)mt * n_nt + nt, g.epoch, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

using GuCfg = Cfg<256, 256, MOE_GU_WAVES_M, MOE_GU_WAVES_N, MOE_BK, MOE_STAGES>;
using Dn256 = Cfg<256, 256, MOE_DN_WAVES_M, MOE_DN_WAVES_N, MOE_BK, MOE_STAGES>;
using Dn128 = Cfg<128, 256, MOE_DN_WAVES_M, MOE_DN_WAVES_N, MOE_BK, MOE_STAGES>;
using Dn64 = Cfg<64, 256, 1, 4, 32, 4>;
using Dn32 = Cfg<32, 256, 1, 4, 64, 3>;

}  // namespace

hipError_t launch_gateup(const PlanLayout& L, const int32_t* ws, const uint16_t* x, const uint16_t* wgu,
                         uint16_t* h, int grid, hipStream_t s) {
  GemmArgs a{ws, x, wgu, h, nullptr, 0u, L.d, L.f, 2 * L.f, L.f};
  hipLaunchKernelGGL((grouped_gemm_kernel<GuCfg, true, false>), dim3(grid), dim3(GuCfg::NT), 0, s, L, a);
  return hipGetLastError();
}

hipError_t launch_down(const PlanLayout& L, const int32_t* ws, const uint16_t* h, const uint16_t* wd,
                       uint16_t* y, uint32_t* flags, uint32_t epoch, int grid, hipStream_t s) {
  GemmArgs a{ws, h, wd, y, flags, epoch, L.f, L.d, L.d, 0};
  switch (L.dn_bm) {
    case 256: hipLaunchKernelGGL((grouped_gemm_kernel<Dn256, false, true>), dim3(grid), dim3(Dn256::NT), 0, s, L, a); break;
    case 128: hipLaunchKernelGGL((grouped_gemm_kernel<Dn128, false, true>), dim3(grid), dim3(Dn128::NT), 0, s, L, a); break;
    case 64: hipLaunchKernelGGL((grouped_gemm_kernel<Dn64, false, true>), dim3(grid), dim3(Dn64::NT), 0, s, L, a); break;
    default: hipLaunchKernelGGL((grouped_gemm_kernel<Dn32, false, true>), dim3(grid), dim3(Dn32::NT), 0, s, L, a); break;
  }
  return hipGetLastError();
}

}  // namespace moe
