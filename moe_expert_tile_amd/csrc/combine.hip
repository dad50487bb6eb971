// Standalone consumer kernel (tile-signal notes, "MoE 计算-通信细粒度重叠：用 Tile 级信号
// 把 All-to-All 藏在 GEMM 背后", §5.2 and §5.3): the consumer body of consume.h on
// its own grid, after the down GEMM (serial mode) or with the flags already
// set (copy-only mode).  The overlapped mode runs the same body inside the
// down-GEMM launch instead.  Also the per-row ablation of the copy (§4.3).
#include "consume.h"

namespace moe {
namespace {

constexpr int kConsumerThreads = 256;

template <bool PIPE>
__global__ __launch_bounds__(kConsumerThreads) void consumer_kernel(PlanLayout L, int32_t* __restrict__ ws,
                                                                   const uint16_t* __restrict__ y,
                                                                   const uint32_t* __restrict__ flags, uint32_t epoch,
                                                                   RecvPtrs recv, CopyCtl cc) {
  __shared__ int s_go;
  consume_segments<kConsumerThreads, PIPE>(L, ws, y, flags, epoch, recv, cc, blockIdx.x, gridDim.x, &s_go);
}

// Per-row ablation of the copy (the alternative the tile-signal notes weigh
// in §4.3: no owner-aligned layout, every output row routed on its own at
// transfer time).  The same remote rows as the consumer's segments, but one
// row per wavefront: each wavefront reads the row's routing (destination
// rank and row) from the plan, waits for its band's flags, and copies the
// row alone.  Rows are enumerated as (remote band, row < tb_M) pairs;
// padding pairs return at once.
__global__ __launch_bounds__(kConsumerThreads) void consumer_rows_kernel(PlanLayout L, int32_t* __restrict__ ws,
                                                                        const uint16_t* __restrict__ y,
                                                                        const uint32_t* __restrict__ flags,
                                                                        uint32_t epoch, RecvPtrs recv,
                                                                        int64_t timeout) {
  int32_t* hdr = ws + L.o_hdr;
  if (__hip_atomic_load(hdr + H_ERROR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  const int n_remote = hdr[H_REMOTE];
  const int32_t* bsrc = ws + L.o_bsrc;
  const int32_t* bval = ws + L.o_bval;
  const int32_t* bdst = ws + L.o_bdst;
  const int32_t* bdoff = ws + L.o_bdoff;
  constexpr int WPB = kConsumerThreads / 64;
  const int lane = threadIdx.x & 63;
  const int64_t n_pairs = (int64_t)n_remote * L.tb_m;
  const int64_t row_bytes = (int64_t)L.d * 2;
  const int tpb = L.dn_tpb;
  for (int64_t i = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6); i < n_pairs; i += (int64_t)gridDim.x * WPB) {
    const int b = (int)(i / L.tb_m), r = (int)(i - (int64_t)b * L.tb_m);
    if (r >= bval[b]) continue;
    // this row's band: every one of its tile flags (head and tail per
    // column tile) must equal epoch
    const uint64_t t0 = wall_clock64();
    int naps = 1;
    for (;;) {
      bool ok = true;
      for (int j = lane; j < 2 * tpb; j += 64)
        ok &= (__hip_atomic_load(flags + (int64_t)b * 2 * tpb + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               epoch);
      if (__ballot(!ok) == 0) break;
      if ((int64_t)(wall_clock64() - t0) > timeout) {
        if (lane == 0)
          __hip_atomic_store(hdr + H_ERROR, 4 /* MOE_ETIMEOUT */, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      for (int z = 0; z < naps; ++z) __builtin_amdgcn_s_sleep(2);
      naps = min(2 * naps, MOE_POLL_MAX_NAPS);
    }
    const __amdgpu_buffer_rsrc_t src = copy_rsrc(y + (int64_t)(bsrc[b] + r) * L.d, row_bytes);
    const __amdgpu_buffer_rsrc_t dst = copy_rsrc(recv.p[bdst[b]] + (int64_t)(bdoff[b] + r) * L.d, row_bytes);
    // 1 KB per wavefront access; up to 8 in flight, all loads before the stores
    constexpr int VPL = 8;
    for (int64_t v0 = 0; v0 < row_bytes; v0 += (int64_t)VPL * 64 * 16) {
      cv4u32 v[VPL];
#pragma unroll
      for (int k = 0; k < VPL; ++k)
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(src, (int)(v0 + (k * 64 + lane) * 16), 0, kAgentLoad);
#pragma unroll
      for (int k = 0; k < VPL; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(v[k], dst, (int)(v0 + (k * 64 + lane) * 16), 0, kStreamStore);
    }
  }
}

}  // namespace

hipError_t launch_consumer_rows(const PlanLayout& L, int32_t* ws, const uint16_t* y, const uint32_t* flags,
                                uint32_t epoch, const RecvPtrs& recv, int64_t timeout_ticks, hipStream_t s) {
  // one wavefront per (band, row) pair of the capacity, at most 65535 workgroups
  const int64_t pairs = (int64_t)L.bands_cap * L.tb_m;
  constexpr int WPB = kConsumerThreads / 64;
  int64_t grid = (pairs + WPB - 1) / WPB;
  grid = grid < 1 ? 1 : (grid > 65535 ? 65535 : grid);
  hipLaunchKernelGGL(consumer_rows_kernel, dim3((unsigned)grid), dim3(kConsumerThreads), 0, s, L, ws, y, flags, epoch,
                     recv, timeout_ticks);
  return hipGetLastError();
}

hipError_t launch_consumer(const PlanLayout& L, int32_t* ws, const uint16_t* y, const uint32_t* flags,
                           uint32_t epoch, const RecvPtrs& recv, const CopyCtl& cc, int grid, hipStream_t s) {
  // a grid of at most one workgroup per CU (a consumer budget) gives each
  // workgroup many units: two in flight per workgroup.  Larger grids (the
  // default, one workgroup per unit) take the variant with half the
  // registers, so more workgroups fit a CU.
  if (grid <= kMaxProducers)
    hipLaunchKernelGGL(consumer_kernel<true>, dim3(grid), dim3(kConsumerThreads), 0, s, L, ws, y, flags, epoch, recv,
                       cc);
  else
    hipLaunchKernelGGL(consumer_kernel<false>, dim3(grid), dim3(kConsumerThreads), 0, s, L, ws, y, flags, epoch, recv,
                       cc);
  return hipGetLastError();
}

}  // namespace moe
