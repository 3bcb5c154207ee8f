// decode_noalloc.hip -- the fixed device scratch of attn_decode_cached_noalloc (declared in
// include/gqa_attn.h, validated and launched in api.hip): cached decode whose split-KV
// partials live in this array instead of a caller workspace, for callers that cannot
// allocate device memory (graph capture, tight serving loops).
//
// In host code the array's name below is only a host-side stand-in; its address on a
// device comes from hipGetSymbolAddress, taken once per device (with that device
// current) and kept.  Only that address is ever handed to the kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gqa_attn.h"
#include "launch.h"

static __device__ __align__(256) char scratch[GQA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_setup;

}  // namespace

namespace gqa {

// Address of the current device's copy of `scratch`; looked up on the first call on
// that device (with that device current), then reused.
int noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GQA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return GQA_EUNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_setup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GQA_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return GQA_OK;
}

}  // namespace gqa
