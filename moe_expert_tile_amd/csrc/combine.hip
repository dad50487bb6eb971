// Standalone consumer kernel (tile-signal notes, "MoE 计算-通信细粒度重叠：用 Tile 级信号
// 把 All-to-All 藏在 GEMM 背后", §5.2 and §5.3): the consumer body of consume.h on
// its own grid, after the down GEMM (serial mode) or with the flags already
// set (copy-only mode).  The overlapped mode runs the same body inside the
// down-GEMM launch instead.
#include "consume.h"

namespace moe {
namespace {

constexpr int kConsumerThreads = 256;

__global__ __launch_bounds__(kConsumerThreads) void consumer_kernel(PlanLayout L, int32_t* __restrict__ ws,
                                                                   const uint16_t* __restrict__ y,
                                                                   const uint32_t* __restrict__ flags, uint32_t epoch,
                                                                   RecvPtrs recv, int64_t timeout) {
  __shared__ int s_go;
  consume_segments<kConsumerThreads>(L, ws, y, flags, epoch, recv, timeout, blockIdx.x, gridDim.x, &s_go);
}

}  // namespace

hipError_t launch_consumer(const PlanLayout& L, int32_t* ws, const uint16_t* y, const uint32_t* flags,
                           uint32_t epoch, const RecvPtrs& recv, int64_t timeout_ticks, int grid, hipStream_t s) {
  hipLaunchKernelGGL(consumer_kernel, dim3(grid), dim3(kConsumerThreads), 0, s, L, ws, y, flags, epoch, recv,
                     timeout_ticks);
  return hipGetLastError();
}

}  // namespace moe
