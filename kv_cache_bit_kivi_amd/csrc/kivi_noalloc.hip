// kivi_noalloc.hip - decode attention without a workspace argument, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that forbid allocation).  The split partials live in a
// file-scope device array of fixed size; each GPU holds its own copy for the
// life of the process, and its address is looked up once per device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/kivi.h"
#include "kivi_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;  // 16 MiB of split partials
constexpr int kMaxDevices = 64;

// The partials of every call on this GPU.  In host code `scratch` names a
// host-side stand-in, not the device copy: kernels and copies take the
// address hipGetSymbolAddress returns (scratch_ptr), never the name.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex lookup_mutex;

// The device address of `scratch` on the current device (looked up on the
// first call on that device, with that device current).
kivi_status device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return kivi::report(KIVI_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return kivi::report(KIVI_ERR_UNSUPPORTED, "device index beyond the 64 the scratch table holds");
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(lookup_mutex);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return kivi::report(KIVI_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
      scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KIVI_OK;
}

}  // namespace

extern "C" kivi_status kivi_decode_attn_noalloc(kivi_cache* cache, const void* q, int32_t num_q_heads,
                                                float softmax_scale, void* out, int32_t out_dtype,
                                                void* stream) {
  void* ws = nullptr;
  const kivi_status st = device_scratch(&ws);
  if (st != KIVI_OK) return st;
  return kivi::decode_attn_bounded(cache, q, num_q_heads, softmax_scale, out, out_dtype, ws, kScratchBytes,
                                   stream);
}
