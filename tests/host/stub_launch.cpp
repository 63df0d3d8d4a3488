// stub_launch.cpp - host-only stand-ins for the kernel launchers and the few
// HIP runtime calls of the host state machine (kivi_api.cpp), so that its
// contract can be exercised without a GPU, under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Test infrastructure: no device is touched.
//
// Each launch is recorded (kind and the arguments that fix its work), and a
// launch can be made to fail: stub_fail_launch(n) makes the n-th launch from
// now return hipErrorLaunchFailure without recording it.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstring>
#include <vector>

#include "../../kv_cache_bit_kivi_amd/csrc/kivi_internal.h"

namespace {
struct Launch {
  int kind;  // 0 pack, 1 window copy, 2 decode (split kernel + merge), 3 read probe
  int nblk, dst_blk0, r_count, r_dst_slot0, ragged;
  int n_quant, n_resid, n_split, n_split_packed, hg, fused_append;
};
std::vector<Launch> g_log;
int g_fail_in = 0;       // launches until the failing one (0: none)
int g_device_ok = 1;     // hipGetDevice succeeds
int g_cus = 256;         // compute units reported
int g_device_calls = 0;  // device queries made

hipError_t take(const Launch& l) {
  if (g_fail_in > 0 && --g_fail_in == 0) return hipErrorLaunchFailure;
  g_log.push_back(l);
  return hipSuccess;
}
}  // namespace

extern "C" {
void stub_reset(void) {
  g_log.clear();
  g_fail_in = 0;
  g_device_ok = 1;
  g_cus = 256;
  g_device_calls = 0;
}
void stub_fail_launch(int n) { g_fail_in = n; }
void stub_device(int ok, int cus) {
  g_device_ok = ok;
  g_cus = cus;
}
int stub_launches(void) { return static_cast<int>(g_log.size()); }
int stub_device_calls(void) { return g_device_calls; }
// fields of launch i: kind, nblk, dst_blk0, r_count, r_dst_slot0, ragged,
// n_quant, n_resid, n_split, n_split_packed, hg, fused_append
void stub_launch(int i, int* f) {
  const Launch& l = g_log.at(static_cast<size_t>(i));
  const int v[12] = {l.kind, l.nblk, l.dst_blk0, l.r_count, l.r_dst_slot0, l.ragged,
                     l.n_quant, l.n_resid, l.n_split, l.n_split_packed, l.hg, l.fused_append};
  std::memcpy(f, v, sizeof v);
}

hipError_t hipGetDevice(int* d) {
  ++g_device_calls;
  if (!g_device_ok) return hipErrorNoDevice;
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = g_cus;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) {
  return e == hipErrorLaunchFailure ? "injected launch failure"
         : e == hipErrorNoDevice    ? "no device (stub)"
                                    : "stub error";
}
}  // extern "C"

namespace kivi {
hipError_t launch_pack(const PackArgs& a, int, int, int, hipStream_t) {
  return take(Launch{0, a.nblk, a.dst_blk0, a.r_count, a.r_dst_slot0, a.ragged, 0, 0, 0, 0, 0, 0});
}
hipError_t launch_resid_copy(const PackArgs& a, int, hipStream_t) {
  return take(Launch{1, 0, 0, a.r_count, a.r_dst_slot0, a.ragged, 0, 0, 0, 0, 0, 0});
}
hipError_t launch_decode(const DecodeArgs& a, int, int, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  return take(Launch{2, 0, 0, 0, 0, a.ragged, a.n_quant, a.n_resid, a.n_split, a.n_split_packed, a.hg,
                     a.k_new != nullptr ? 1 : 0});
}
hipError_t launch_stream_read(const void*, size_t, uint32_t*, int, hipStream_t) {
  return take(Launch{3, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0});
}
}  // namespace kivi
