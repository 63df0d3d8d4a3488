// kivi_probe.hip - a streaming-read probe: the HBM read rate a plain kernel
// reaches on this device, the practical ceiling against which the decode's
// rate (a kernel that only streams the packed cache once) is compared.
//
// Each workgroup of 256 threads reads one contiguous chunk of the source with
// 16-byte non-temporal loads, four in flight per thread, and every thread
// writes the XOR of what it read to the sink, so that no load can be elided.
#include <hip/hip_runtime.h>

#include "kivi_internal.h"

namespace kivi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(const u32x4& v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__global__ __launch_bounds__(256) void stream_read(const u32x4* src, size_t n16, uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;  // 16-byte words per workgroup
  const size_t b = static_cast<size_t>(blockIdx.x) * per;
  const size_t e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0;
  size_t i = b + threadIdx.x;
  for (; i + 3 * 256 < e; i += 4 * 256) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
    acc ^= fold(v0) ^ fold(v1) ^ fold(v2) ^ fold(v3);
  }
  for (; i < e; i += 256) acc ^= fold(__builtin_nontemporal_load(src + i));
  sink[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read, dim3(workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace kivi
