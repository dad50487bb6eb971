// moe_expert_combine_noalloc: moe_expert_combine for callers that cannot
// allocate device memory.  Its kernels' scratch -- the partial sums of the
// GEMMs' K-split tails, their tile counters, and the copy-claim counters of
// the overlapped launch -- lives in one static device array per GPU instead
// of the plan workspace.
#include "moe_internal.h"

#include <mutex>

namespace moe {
namespace {

constexpr int kStaticSkSlots = 256;                        // partial-sum slots of 256x256 fp32 (64 MiB)
constexpr size_t kCtrBytes = 2 * kMaxProducers * 8;        // uint64 tile counters, gate/up and down
constexpr size_t kClaimOff = kCtrBytes;                    // two int32 claim counters (256 bytes kept)
constexpr size_t kLinkOff = kClaimOff + 256;               // uint64 link busy-until time per destination
constexpr size_t kGreadyOff = kLinkOff + kMaxWorld * 8;    // uint64 group ready counters
constexpr size_t kPartOff = kGreadyOff + kMaxGroups * 8;   // partial sums
constexpr size_t kScratchBytes = kPartOff + (size_t)kStaticSkSlots * 256 * 256 * 4;
static_assert(kPartOff % 256 == 0, "aligned partial sums");

// The array itself.  In host code its name is a host-side stand-in, not a
// device address: only the address hipGetSymbolAddress returns for the
// current device is used below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 16;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// the device address of `scratch` on device `dev` (the current device),
// looked up once per device
int static_scratch(int dev, Scratch* out) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  void* p;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return MOE_EHIP;
      g_scratch[dev] = q;
    }
    p = g_scratch[dev];
  }
  char* base = (char*)p;
  out->sk_ctr = (uint64_t*)base;
  out->claim = (int32_t*)(base + kClaimOff);
  out->link_free = (uint64_t*)(base + kLinkOff);
  out->gready = (uint64_t*)(base + kGreadyOff);
  out->sk_part = (float*)(base + kPartOff);
  out->sk_slots = kStaticSkSlots;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_expert_combine_noalloc(const moe_shape* s, const void* plan_ws, const uint16_t* x_layout,
                                          const uint16_t* w_gate_up, const uint16_t* w_down, uint16_t* h,
                                          uint16_t* y, uint32_t* flags, uint32_t epoch, uint16_t* const* recv,
                                          const moe_combine_opts* opts, void* stream) {
  return moe::combine_impl(s, plan_ws, x_layout, w_gate_up, w_down, h, y, flags, epoch, recv, opts, stream,
                           moe::static_scratch);
}
