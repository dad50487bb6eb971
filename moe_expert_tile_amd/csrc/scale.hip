// Scale: step 5 of the distributed MoE forward in the tile-signal notes
// ("MoE 计算-通信细粒度重叠：用 Tile 级信号把 All-to-All 藏在 GEMM 背后", §2.2; §2.1: the
// layer output is the gate-weighted sum of the k selected experts' outputs).
//   out[t] = bf16( sum_{j<k} w[t][j] * recv[pos[t][j]] ), fp32, j ascending.
// One wavefront per run of 256 16-byte output vectors of a token: each lane
// keeps the row loads of 4 slots in flight at once (16 loads, each a
// contiguous 1 KB access across the wavefront), fp32 fused multiply-adds in
// slot order, one round-to-nearest-even conversion per value, 16-byte
// stores.  The returned rows are read
// once, mostly from HBM, with nontemporal loads: measured 4-9% faster in the
// step and 3-8% with a cold Infinity Cache, though 10% slower when the rows
// are still in that cache.
#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;   // raw buffer access: data format 32, other fields zero
constexpr int kNontemporal = 2;         // nt cache-policy bit

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__global__ __launch_bounds__(256) void scale_kernel(PlanLayout L, const int32_t* __restrict__ ws,
                                                   const uint4* __restrict__ recv, const float* __restrict__ w,
                                                   uint4* __restrict__ out) {
  if (ws[L.o_hdr + H_ERROR] != 0) return;
  const int32_t* pos = ws + L.o_pos;
  const int k = L.k;
  const int64_t vec = L.d / 8;
  // a wavefront takes a run of 64*VPT vectors of one token's row; lane l
  // handles vectors l, l+64, l+128, l+192 of the run, so each of its VPT*k
  // row loads is a contiguous 1 KB access across the wavefront
  constexpr int VPT = 4, RUN = 64 * VPT;
  const int64_t runs = (vec + RUN - 1) / RUN;
  const int64_t total_waves = (int64_t)L.T_r * runs;
  const int lane = threadIdx.x & 63;
  const int64_t wpb = blockDim.x >> 6;
  // the wavefront's run, token and slots are wave-uniform: the slot table
  // and the weights are read with scalar loads, and each row's buffer
  // descriptor lives in scalar registers
  const int64_t wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  for (int64_t wv = (int64_t)blockIdx.x * wpb + wave; wv < total_waves; wv += (int64_t)gridDim.x * wpb) {
    const int64_t t = wv / runs;
    const int64_t v0 = (wv - t * runs) * RUN + lane;
    float acc[VPT][8];
#pragma unroll
    for (int q = 0; q < VPT; ++q)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[q][c] = 0.f;
    // KC slots at a time: all their row loads are issued before the first
    // multiply-add, so each lane keeps KC * VPT loads in flight; the sums
    // still run over the slots in ascending order
    constexpr int KC = 4;
    for (int j0 = 0; j0 < k; j0 += KC) {
      v4u32 x[KC][VPT];
      float wj[KC];
      int pj[KC];
#pragma unroll
      for (int jj = 0; jj < KC; ++jj) {
        const int j = min(j0 + jj, k - 1);
        wj[jj] = w[t * k + j];
        pj[jj] = pos[t * k + j];
      }
#pragma unroll
      for (int jj = 0; jj < KC; ++jj) {
        // one row: loads past its end (a ragged last run) read zeros; a slot
        // past k gets an empty descriptor (its loads return zeros and are
        // not used), so the loads need no branch
        const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(recv + (int64_t)pj[jj] * vec), (short)0, j0 + jj < k ? (int)(vec * 16) : 0, kBufWord3);
#pragma unroll
        for (int q = 0; q < VPT; ++q)
          x[jj][q] = __builtin_amdgcn_raw_buffer_load_b128(row, (int)((v0 + 64 * q) * 16), 0, kNontemporal);
      }
#pragma unroll
      for (int jj = 0; jj < KC; ++jj) {
        if (j0 + jj < k) {
#pragma unroll
          for (int q = 0; q < VPT; ++q) {
            const v4u32 v = x[jj][q];
            const float wt = wj[jj];
            acc[q][0] = fmaf(wt, bf_lo(v[0]), acc[q][0]);
            acc[q][1] = fmaf(wt, bf_hi(v[0]), acc[q][1]);
            acc[q][2] = fmaf(wt, bf_lo(v[1]), acc[q][2]);
            acc[q][3] = fmaf(wt, bf_hi(v[1]), acc[q][3]);
            acc[q][4] = fmaf(wt, bf_lo(v[2]), acc[q][4]);
            acc[q][5] = fmaf(wt, bf_hi(v[2]), acc[q][5]);
            acc[q][6] = fmaf(wt, bf_lo(v[3]), acc[q][6]);
            acc[q][7] = fmaf(wt, bf_hi(v[3]), acc[q][7]);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      if (v0 + 64 * q < vec) {
        uint4 o;
        o.x = pack2(acc[q][0], acc[q][1]);
        o.y = pack2(acc[q][2], acc[q][3]);
        o.z = pack2(acc[q][4], acc[q][5]);
        o.w = pack2(acc[q][6], acc[q][7]);
        out[t * vec + v0 + 64 * q] = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_scale(const PlanLayout& L, const int32_t* ws, const uint16_t* recv_self, const float* topk_w,
                        uint16_t* out, hipStream_t s) {
  const int64_t runs = (L.d / 8 + 255) / 256;            // 256-vector runs per row, one wavefront each
  const int64_t waves = (int64_t)L.T_r * runs;
  if (waves == 0) return hipSuccess;
  int64_t grid = (waves + 3) / 4;
  if (grid > 16384) grid = 16384;
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)grid), dim3(256), 0, s, L, ws, (const uint4*)recv_self, topk_w,
                     (uint4*)out);
  return hipGetLastError();
}

}  // namespace moe
