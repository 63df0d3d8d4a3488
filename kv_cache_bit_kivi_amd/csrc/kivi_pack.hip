// kivi_pack.hip - quantize and bit-pack blocks of G = 32 tokens (keys per
// channel, values per token) and copy tokens into the residual window.
//
// Method: page "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide", "The
// Three Structural Innovations of KIVI" (items 1-3) and "Step 1" (min/max
// scale, half-to-even rounding, clamp); page "KV cache quantization with KIVI
// INT2 setup guide", "KIVI: Per-Channel Key, Per-Token Value Quantization
// Explained" (G = 32, R = 128).  Every binary32 step is a single correctly
// rounded operation (built with -ffp-contract=off, IEEE division, denormals
// kept), so codes are reproducible bit for bit.
//
// One workgroup (256 threads, 4 waves) owns one block of one (batch, kv
// head) unit: it stages the 32 x 128 key and value tiles in LDS with 16-byte
// coalesced loads, reduces the group minima/maxima, then writes whole 32-bit
// code words with coalesced stores.  Extra workgroups of the same launch copy
// the trailing tokens into the residual window.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int G = kGroup;
constexpr int D = kHeadDim;
constexpr int RS = D + 8;  // LDS row stride in 16-bit elements (272 bytes)

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  } else {
    return __half2float(__ushort_as_half(h));
  }
}

// fp16 bit pattern of a binary32 value, nearest-even; zero is stored as +0.
__device__ __forceinline__ uint16_t f16_bits_canon(float f) {
  return f == 0.0f ? uint16_t(0) : __half_as_ushort(__float2half_rn(f));
}

// Per-group constants: minimum, binary32 scale s = (max - min) / qmax and the
// reciprocal used by the fast path.  rcp = 0 when s == 0 (every code is then
// 0) and NaN when s is so small that RN(1/s) could leave the normal range
// (every code then takes the exact division).
template <int QMAX>
__device__ __forceinline__ void group_consts(float mn, float mx, float& s, float& rcp) {
  s = (mx - mn) / static_cast<float>(QMAX);
  if (s == 0.0f) {
    rcp = 0.0f;
  } else if (s < 0x1p-100f) {
    rcp = __builtin_nanf("");
  } else {
    rcp = 1.0f / s;
  }
}

// Code of x: clamp(rne(RN(RN(x - mn) / s)), 0, qmax).
// Fast path y = RN(d * rcp).  With rcp = RN(1/s), |y - RN(d / s)| is below
// 3 * 2^-24 * |d / s| <= 3 * 2^-24 * 16 < 2^-18, so rounding y to an integer
// gives the same result unless y lies within 2^-18 of a half-integer; those
// rare elements (and NaN from the tiny-scale case) redo the exact division.
template <int QMAX>
__device__ __forceinline__ uint32_t quant_code(float x, float mn, float s, float rcp) {
  const float d = x - mn;
  const float y = d * rcp;
  float r = rintf(y);
  const float f = y - r;  // exact: y and r are within 1/2 of each other
  if (!(fabsf(f) <= 0.49999237060546875f)) {  // 0.5 - 2^-17
    r = rintf(d / s);
  }
  r = fminf(fmaxf(r, 0.0f), static_cast<float>(QMAX));
  return static_cast<uint32_t>(r);
}

// Bit offset of code i in a word: even codes low half-word, odd codes high.
template <int BITS>
__device__ __forceinline__ int code_shift(int i) {
  return BITS * (i >> 1) + 16 * (i & 1);
}

template <int KB, int VB, bool BF16>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  constexpr int QK = (1 << KB) - 1, QV = (1 << VB) - 1;
  constexpr int PK = 32 / KB;  // key codes (channels) per word
  constexpr int KW = D / PK;   // key words per token
  constexpr int PV = 32 / VB;  // value codes (rows) per word
  constexpr int VW = G / PV;   // value words per (block, channel)

  __shared__ __align__(16) uint16_t kt[G * RS];
  __shared__ __align__(16) uint16_t vt[G * RS];
  __shared__ float kmn[D], ksc[D], krc[D];
  __shared__ float vmn[4 * G], vsc[4 * G], vrc[4 * G];  // index m * G + row

  const int tid = threadIdx.x;
  const int item = blockIdx.x;
  const long long u = blockIdx.y;

  if (item >= a.nblk) {
    // ---- residual-window copy: 32 tokens per workgroup
    const int t0 = (item - a.nblk) * G;
    const int n = min(G, a.r_count - t0);
    for (int c = tid; c < n * (D / 8); c += 256) {
      const int t = t0 + c / (D / 8), col = (c % (D / 8)) * 8;
      const long long src = u * a.r_src_unit_stride + (long long)(a.r_src_tok0 + t) * D + col;
      const long long dst = (u * a.R + a.r_dst_slot0 + t) * D + col;
      *reinterpret_cast<uint4*>(a.k_resid + dst) = *reinterpret_cast<const uint4*>(a.rk_src + src);
      *reinterpret_cast<uint4*>(a.v_resid + dst) = *reinterpret_cast<const uint4*>(a.rv_src + src);
    }
    return;
  }

  // ---- stage the key and value tiles of this block
  constexpr BlockLayout BL = block_layout(KB, VB);
  const int blk = item;
  const int gblk = a.dst_blk0 + blk;
  uint8_t* const rec = a.blocks + (u * a.nb + gblk) * BL.bytes;  // this block's record
  {
    const long long base = u * a.src_unit_stride + (long long)(a.src_tok0 + blk * G) * D;
    for (int c = tid; c < G * D / 8; c += 256) {
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const uint4 kx = *reinterpret_cast<const uint4*>(a.k_src + base + row * D + col);
      const uint4 vx = *reinterpret_cast<const uint4*>(a.v_src + base + row * D + col);
      *reinterpret_cast<uint4*>(&kt[row * RS + col]) = kx;
      *reinterpret_cast<uint4*>(&vt[row * RS + col]) = vx;
    }
  }
  __syncthreads();

  // ---- group statistics
  if (tid < D) {
    // key group: channel d over the G rows of the block
    const int d = tid;
    float mn = to_f32<BF16>(kt[d]), mx = mn;
    for (int t = 1; t < G; ++t) {
      const float x = to_f32<BF16>(kt[t * RS + d]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    float s, rcp;
    group_consts<QK>(mn, mx, s, rcp);
    kmn[d] = mn;
    ksc[d] = s;
    krc[d] = rcp;
    reinterpret_cast<uint16_t*>(rec + BL.k_scale)[d] = f16_bits_canon(s);
    reinterpret_cast<uint16_t*>(rec + BL.k_zero)[d] = f16_bits_canon(mn);
  } else {
    // value group: row t, channels m*G .. m*G+G-1; thread index m*G + t
    const int i = tid - D;
    const int m = i / G, t = i % G;
    const uint16_t* row = &vt[t * RS + m * G];
    float mn = to_f32<BF16>(row[0]), mx = mn;
    for (int c = 1; c < G; ++c) {
      const float x = to_f32<BF16>(row[c]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    float s, rcp;
    group_consts<QV>(mn, mx, s, rcp);
    vmn[i] = mn;
    vsc[i] = s;
    vrc[i] = rcp;
    reinterpret_cast<uint16_t*>(rec + BL.v_scale)[i] = f16_bits_canon(s);  // [m][row]
    reinterpret_cast<uint16_t*>(rec + BL.v_zero)[i] = f16_bits_canon(mn);
  }
  __syncthreads();

  // ---- key code words: token row t, word w holds channels w*PK .. w*PK+PK-1
  for (int wi = tid; wi < G * KW; wi += 256) {
    const int t = wi / KW, w = wi % KW;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      const int d = w * PK + i;
      const uint32_t c = quant_code<QK>(to_f32<BF16>(kt[t * RS + d]), kmn[d], ksc[d], krc[d]);
      word |= c << code_shift<KB>(i);
    }
    reinterpret_cast<uint32_t*>(rec + BL.k_codes)[t * KW + w] = word;
  }

  // ---- value code words: channel d, word w holds rows w*PV .. w*PV+PV-1;
  // word-major, so consecutive threads write consecutive channels
  for (int wi = tid; wi < D * VW; wi += 256) {
    const int w = wi / D, d = wi % D;
    const int m = d / G;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < PV; ++i) {
      const int t = w * PV + i;
      const int si = m * G + t;
      const uint32_t c = quant_code<QV>(to_f32<BF16>(vt[t * RS + d]), vmn[si], vsc[si], vrc[si]);
      word |= c << code_shift<VB>(i);
    }
    reinterpret_cast<uint32_t*>(rec + BL.v_codes)[w * D + d] = word;
  }
}

template <int KB, int VB, bool BF16>
hipError_t launch_pack_t(const PackArgs& a, hipStream_t stream) {
  const int items = a.nblk + (a.r_count + G - 1) / G;
  if (items == 0) return hipSuccess;
  dim3 grid(items, a.units);
  hipLaunchKernelGGL((pack_kernel<KB, VB, BF16>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, int k_bits, int v_bits, int kv_dtype,
                       hipStream_t stream) {
  const bool bf = kv_dtype == 1;
#define KIVI_PACK_CASE(KB, VB)                                                  \
  if (k_bits == KB && v_bits == VB)                                             \
    return bf ? launch_pack_t<KB, VB, true>(a, stream) : launch_pack_t<KB, VB, false>(a, stream);
  KIVI_PACK_CASE(2, 2)
  KIVI_PACK_CASE(2, 4)
  KIVI_PACK_CASE(4, 2)
  KIVI_PACK_CASE(4, 4)
#undef KIVI_PACK_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_resid_copy(const PackArgs& a, int kv_dtype, hipStream_t stream) {
  (void)kv_dtype;  // a bit copy: the element type does not matter
  PackArgs c = a;
  c.nblk = 0;
  return launch_pack_t<2, 2, false>(c, stream);
}

}  // namespace kivi
