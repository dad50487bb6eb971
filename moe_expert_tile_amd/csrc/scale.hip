// Scale: step 5 of the distributed MoE forward in the tile-signal notes
// ("MoE 计算-通信细粒度重叠：用 Tile 级信号把 All-to-All 藏在 GEMM 背后", §2.2; §2.1: the
// layer output is the gate-weighted sum of the k selected experts' outputs).
//   out[t] = bf16( sum_{j<k} w[t][j] * recv[pos[t][j]] ), fp32, j ascending.
// One thread per 16-byte output vector: k coalesced 16-byte row loads, fp32
// fused multiply-adds, one round-to-nearest-even conversion, one 16-byte store.
#include "moe_internal.h"

namespace moe {
namespace {

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
  const int64_t total = (int64_t)L.T_r * vec;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / vec, v = i - t * vec;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const float wj = w[t * k + j];
      const uint4 x = recv[(int64_t)pos[t * k + j] * vec + v];
      acc[0] = fmaf(wj, bf_lo(x.x), acc[0]);
      acc[1] = fmaf(wj, bf_hi(x.x), acc[1]);
      acc[2] = fmaf(wj, bf_lo(x.y), acc[2]);
      acc[3] = fmaf(wj, bf_hi(x.y), acc[3]);
      acc[4] = fmaf(wj, bf_lo(x.z), acc[4]);
      acc[5] = fmaf(wj, bf_hi(x.z), acc[5]);
      acc[6] = fmaf(wj, bf_lo(x.w), acc[6]);
      acc[7] = fmaf(wj, bf_hi(x.w), acc[7]);
    }
    uint4 o;
    o.x = pack2(acc[0], acc[1]);
    o.y = pack2(acc[2], acc[3]);
    o.z = pack2(acc[4], acc[5]);
    o.w = pack2(acc[6], acc[7]);
    out[i] = o;
  }
}

}  // namespace

hipError_t launch_scale(const PlanLayout& L, const int32_t* ws, const uint16_t* recv_self, const float* topk_w,
                        uint16_t* out, hipStream_t s) {
  const int64_t total = (int64_t)L.T_r * (L.d / 8);
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 16384) grid = 16384;
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)grid), dim3(256), 0, s, L, ws, (const uint4*)recv_self, topk_w,
                     (uint4*)out);
  return hipGetLastError();
}

}  // namespace moe
