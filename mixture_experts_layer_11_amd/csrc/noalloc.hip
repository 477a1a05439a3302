// moe_forward_noalloc: moe_forward with the library's own device scratch
// instead of a caller workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The scratch is one file-scope device array per GPU,
// kNoAllocScratchBytes long, held by each GPU the library runs on until the
// process ends.  Its device address comes from hipGetSymbolAddress, once per
// device on the entry point's first call there (the array's name in host
// code is only a host-side stand-in).  Nothing in it needs to start at zero:
// moe_forward overwrites every workspace byte it reads.  Calls that overlap
// on one GPU share the array and race.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "kernels.h"

namespace {

constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};   // scratch's device address on each device

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_params* p, int64_t T, const void* x,
                                          const moe_weights* w, void* y, int32_t* topk_idx,
                                          float* topk_w, int32_t* counts, void* stream) {
  size_t need = 0;
  moe_status s = moe_workspace_size(p, T, &need);   // validates p and T (host only)
  if (s != MOE_OK) return s;
  if (need > kNoAllocScratchBytes) {
    moe::set_last_error(
        ("moe_forward_noalloc: the workspace for T=" + std::to_string(T) + " is " +
         std::to_string(need) + " bytes, above its fixed scratch of " +
         std::to_string(kNoAllocScratchBytes) + " bytes; use moe_forward with a workspace")
            .c_str());
    return MOE_ERR_UNSUPPORTED;
  }
  if (T == 0) return moe_forward(p, T, x, w, y, topk_idx, topk_w, counts, nullptr, 0, stream);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    moe::set_last_error("moe_forward_noalloc: no current HIP device in range");
    return MOE_ERR_HIP;
  }
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_ptr[dev] == nullptr) {
      e = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_ptr[dev] = nullptr;
        moe::set_last_error((std::string("moe_forward_noalloc: hipGetSymbolAddress: ") +
                                   hipGetErrorString(e)).c_str());
        return MOE_ERR_HIP;
      }
    }
    ptr = g_ptr[dev];
  }
  return moe_forward(p, T, x, w, y, topk_idx, topk_w, counts, ptr, kNoAllocScratchBytes, stream);
}
