// kivi_decode.hip - the cross-split merge of split-K decode attention, and
// the launcher of the decode step (split kernel, then merge).
//
// Method: decode attention must read the whole cache for every new token, so
// it is bound by memory traffic; the token axis is split across many
// workgroups (page "KV-Cache Quantization: I Ran the Experiments",
// "Component 1").  Each split keeps an online softmax in base 2 (q is
// pre-scaled by softmax_scale * log2 e) and writes (m, l, o[D]) per query
// head; the merge combines the splits exactly:
//   M = max m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int D = kHeadDim;

// ---------------------------------------------------------------------------
// Merge of the per-split partial softmax states; one workgroup per (b, j):
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// The split weights are computed once, in parallel, and the D outputs then
// stream the o_s with several loads in flight per thread.
template <int OUT>
__global__ __launch_bounds__(D) void decode_merge(DecodeArgs a) {
  constexpr int kPre = 16;  // splits whose o_s values are loaded up front
  __shared__ float wsh[kMaxSplits];
  __shared__ float red[2][D / 64];
  const long long bj = (long long)a.seq0 * a.Hq + blockIdx.x;  // seq0 = 0 unless ragged
  const int d = threadIdx.x, lane = d & 63, wv = d >> 6;
  const int ns = a.n_split;
  const float* P = a.partial + bj * ns * (D + 2);
  // every load of the first kPre splits is issued before any is used: one
  // memory round trip for (m, l) and those o_s together
  float ms[kMaxSplits / D], ls[kMaxSplits / D], xo[kPre];
#pragma unroll
  for (int k = 0; k < kMaxSplits / D; ++k) {
    const int s = d + k * D;
    ms[k] = s < ns ? P[s * (D + 2)] : -INFINITY;
    ls[k] = s < ns ? P[s * (D + 2) + 1] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < kPre; ++k) xo[k] = k < ns ? P[k * (D + 2) + 2 + d] : 0.0f;
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMaxSplits / D; ++k) mx = fmaxf(mx, ms[k]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[0][wv] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int w = 1; w < D / 64; ++w) M = fmaxf(M, red[0][w]);
  float lsum = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxSplits / D; ++k) {
    const int s = d + k * D;
    if (s < ns) {
      // a split that saw no token has m = -inf and weight 0
      const float w = ms[k] == -INFINITY ? 0.0f : exp2f(ms[k] - M);
      wsh[s] = w;
      lsum = fmaf(w, ls[k], lsum);
    }
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  if (lane == 0) red[1][wv] = lsum;
  __syncthreads();
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < D / 64; ++w) L += red[1][w];
  float O = 0.0f;
#pragma unroll
  for (int k = 0; k < kPre; ++k)
    if (k < ns) O = fmaf(wsh[k], xo[k], O);
  int s = kPre;
  for (; s + 8 <= ns; s += 8) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = P[(s + k) * (D + 2) + 2 + d];
#pragma unroll
    for (int k = 0; k < 8; ++k) O = fmaf(wsh[s + k], x[k], O);
  }
  for (; s < ns; ++s) O = fmaf(wsh[s], P[s * (D + 2) + 2 + d], O);
  // a sequence without tokens (ragged caches only) gets zeros
  const float r = L > 0.0f ? O / L : 0.0f;
  if constexpr (OUT == 2) {
    static_cast<float*>(a.out)[bj * D + d] = r;
  } else if constexpr (OUT == 1) {
    static_cast<__hip_bfloat16*>(a.out)[bj * D + d] = __float2bfloat16(r);
  } else {
    static_cast<__half*>(a.out)[bj * D + d] = __float2half_rn(r);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int k_bits, int v_bits, int kv_dtype,
                         int out_dtype, hipStream_t stream,
                         hipEvent_t split_begin, hipEvent_t split_end) {
  hipError_t e;
  if (split_begin && (e = hipEventRecord(split_begin, stream)) != hipSuccess) return e;
  if ((e = launch_decode_mfma(a, k_bits, v_bits, kv_dtype, stream)) != hipSuccess) return e;
  if (split_end && (e = hipEventRecord(split_end, stream)) != hipSuccess) return e;
  dim3 grid(a.B * a.Hq);
  switch (out_dtype) {
    case 0: hipLaunchKernelGGL(decode_merge<0>, grid, dim3(D), 0, stream, a); break;
    case 1: hipLaunchKernelGGL(decode_merge<1>, grid, dim3(D), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_merge<2>, grid, dim3(D), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kivi
