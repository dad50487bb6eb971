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

constexpr int BK = 64;       // K elements per stage: 128-byte rows, 8 chunks of 16 B
constexpr int kGroupM = 8;   // row tiles per column sweep

template <int BM_, int BN_, int WAVES_M, int WAVES_N, bool SWIGLU>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int FM = WM / 32;
  static constexpr int FN = WN / 32;
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BN * BK;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * 2;
  static constexpr int A_LOADS = BM / 8 / NW;  // 1 KB wave loads per stage
  static constexpr int B_LOADS = BN / 8 / NW;
  static_assert(NW == 4, "four wavefronts per workgroup");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "whole wave loads");
  static_assert(!SWIGLU || (FN % 2 == 0), "gate/up pairs");
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

// Tile t of a (n_mt x n_nt) grid in grouped order -> (mt, nt).
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
__device__ __forceinline__ void issue_stage(lds_void_t* lds_stage, const uint16_t* const (&a_src)[C::A_LOADS],
                                            const uint16_t* const (&b_src)[C::B_LOADS], int k0, int wave) {
  // wave `wave` loads rows [8q, 8q+8) for q = wave, wave + NW, ...; the lane
  // pointers already include the swizzled chunk
  char* base = (char*)lds_stage;
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int q = wave + i * C::NW;
    __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + k0), (lds_void_t*)(base + q * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int q = wave + i * C::NW;
    __builtin_amdgcn_global_load_lds((const void*)(b_src[i] + k0), (lds_void_t*)(base + C::A_ELEMS * 2 + q * 1024),
                                     16, 0, 0);
  }
}

template <class C, bool SWIGLU, bool FLAGS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(PlanLayout L, GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * C::STAGE_ELEMS];
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
  const int KT = g.K / BK;
  const int32_t* rowoff = g.ws + L.o_rowoff;

  // lane-invariant pieces of the load addresses: lane l fills LDS row 8q + l/8,
  // physical chunk l%8, which holds logical chunk (l%8) ^ (l/8)
  const int ld_row = lane >> 3;
  const int ld_chunk = (lane & 7) ^ (lane >> 3);

  for (int t = slot; t < total; t += G) {
    int mt, nt;
    decode_tile(t, n_mt, n_nt, mt, nt);
    int e, row0, row_end;
    if constexpr (SWIGLU) {
      row0 = g.ws[L.o_gumt_row + mt];
      e = g.ws[L.o_gumt_exp + mt];
    } else {
      const int band = mt / L.dn_sub;
      e = g.ws[L.o_bexp + band];
      row0 = g.ws[L.o_bsrc + band] + (mt - band * L.dn_sub) * C::BM;
    }
    row_end = rowoff[e + 1];

    const uint16_t* a_src[C::A_LOADS];
    const uint16_t* b_src[C::B_LOADS];
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int r = (wave + i * C::NW) * 8 + ld_row;
      const int row = min(row0 + r, row_end - 1);
      a_src[i] = g.a + (int64_t)row * g.K + ld_chunk * 8;
    }
    const uint16_t* wexp = g.w + (int64_t)e * g.w_rows * g.K;
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      const int r = (wave + i * C::NW) * 8 + ld_row;
      int wrow;
      if constexpr (SWIGLU) {
        constexpr int HB = C::BN / 2;
        wrow = (r < HB) ? (nt * HB + r) : (g.half + nt * HB + (r - HB));
      } else {
        wrow = nt * C::BN + r;
      }
      b_src[i] = wexp + (int64_t)wrow * g.K + ld_chunk * 8;
    }

    f32x16 acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    issue_stage<C>((lds_void_t*)lds, a_src, b_src, 0, wave);
    wait_vm0();
    __syncthreads();

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
    const int lrow = lane & 31, lhalf = lane >> 5, lsw = lane & 7;

    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT)
        issue_stage<C>((lds_void_t*)(lds + (cur ^ 1) * C::STAGE_ELEMS), a_src, b_src, (kt + 1) * BK, wave);
      const uint16_t* sa = lds + cur * C::STAGE_ELEMS;
      const uint16_t* sb = sa + C::A_ELEMS;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int phys = ((2 * kk + lhalf) ^ lsw) * 8;
        bf16x8 pw[C::FN], px[C::FM];
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
          pw[i] = *(const bf16x8*)(sb + (prow[i] + lrow) * BK + phys);
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
          px[j] = *(const bf16x8*)(sa + (wave_m * C::WM + 32 * j + lrow) * BK + phys);
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
          for (int j = 0; j < C::FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pw[i], px[j], acc[i][j], 0, 0, 0);
      }
      wait_vm0();
      __syncthreads();
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
      if constexpr (FLAGS) {
        // every wave's stores have reached L2; then one release at agent scope
        // (L2 write-back) before the flag of this tile is set
        wait_vm0();
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

using GuCfg = Cfg<256, 256, 2, 2, true>;
using Dn256 = Cfg<256, 256, 2, 2, false>;
using Dn128 = Cfg<128, 256, 2, 2, false>;
using Dn64 = Cfg<64, 256, 1, 4, false>;
using Dn32 = Cfg<32, 256, 1, 4, false>;

}  // namespace

hipError_t launch_gateup(const PlanLayout& L, const int32_t* ws, const uint16_t* x, const uint16_t* wgu,
                         uint16_t* h, int grid, hipStream_t s) {
  GemmArgs a{ws, x, wgu, h, nullptr, 0u, L.d, L.f, 2 * L.f, L.f};
  hipLaunchKernelGGL((grouped_gemm_kernel<GuCfg, true, false>), dim3(grid), dim3(256), 0, s, L, a);
  return hipGetLastError();
}

hipError_t launch_down(const PlanLayout& L, const int32_t* ws, const uint16_t* h, const uint16_t* wd,
                       uint16_t* y, uint32_t* flags, uint32_t epoch, int grid, hipStream_t s) {
  GemmArgs a{ws, h, wd, y, flags, epoch, L.f, L.d, L.d, 0};
  switch (L.dn_bm) {
    case 256: hipLaunchKernelGGL((grouped_gemm_kernel<Dn256, false, true>), dim3(grid), dim3(256), 0, s, L, a); break;
    case 128: hipLaunchKernelGGL((grouped_gemm_kernel<Dn128, false, true>), dim3(grid), dim3(256), 0, s, L, a); break;
    case 64: hipLaunchKernelGGL((grouped_gemm_kernel<Dn64, false, true>), dim3(grid), dim3(256), 0, s, L, a); break;
    default: hipLaunchKernelGGL((grouped_gemm_kernel<Dn32, false, true>), dim3(grid), dim3(256), 0, s, L, a); break;
  }
  return hipGetLastError();
}

}  // namespace moe
