// decode_noalloc.hip -- attn_decode_cached_noalloc: cached decode whose split-KV partials
// live in a fixed device array of the library instead of a caller workspace, for callers
// that cannot allocate device memory (graph capture, tight serving loops).
//
// In host code the array's name below is only a host-side stand-in; its address on a
// device comes from hipGetSymbolAddress, taken once per device (with that device
// current) and kept.  Only that address is ever handed to the kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gqa_attn.h"

static __device__ __align__(256) char scratch[GQA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_setup;

// Address of the current device's copy of `scratch`; looked up on the first call on
// that device, then reused.
int scratch_on_current_device(void** ptr) {
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

}  // namespace

extern "C" int attn_decode_cached_noalloc(const void* q, const void* kcache, const void* vcache,
                                          float* out, int newTokens, int totalLen, int startPos,
                                          int Hq, int Hkv, int d_h, int B, int dtype,
                                          void* stream) {
  // the plan depends on the shape only (0 for shapes attn_decode_cached rejects, which
  // it then reports itself)
  const size_t need = attn_decode_workspace_bytes(B, newTokens, totalLen, Hq, Hkv, d_h, dtype);
  if (need > GQA_NOALLOC_SCRATCH_BYTES) return GQA_ESCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_on_current_device(&ws);
    if (rc != GQA_OK) return rc;
  }
  return attn_decode_cached(q, kcache, vcache, out, newTokens, totalLen, startPos, Hq, Hkv, d_h, B,
                            dtype, ws, need > 0 ? GQA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
