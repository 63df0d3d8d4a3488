// kivi_pack_core.h - quantize and bit-pack one block of G = 32 or 64 tokens of
// one (batch, kv head) unit: keys per channel, values per token.  Shared by
// the pack kernel (256 threads per block) and the window flush inside the
// decode kernel (128 threads).
//
// Method: page "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide", "The
// Three Structural Innovations of KIVI" (items 1-3) and "Step 1" (min/max
// scale, half-to-even rounding, clamp); page "KV cache quantization with KIVI
// INT2 setup guide", "KIVI: Per-Channel Key, Per-Token Value Quantization
// Explained" (G = 32, R = 128).  Every binary32 step is a single correctly
// rounded operation (no contraction in these functions, IEEE division,
// denormals kept), so codes are reproducible bit for bit whichever kernel
// runs them.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace packcore {

constexpr int D = kHeadDim;
constexpr int RS = D + 8;  // LDS row stride in 16-bit elements (272 bytes)

// Streaming accesses: the pack reads each input byte once and writes each
// record byte once, so both go out with the non-temporal hint.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <typename T>
__device__ __forceinline__ void store_stream(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}
__device__ __forceinline__ void store_stream2(uint32_t* p, uint32_t x, uint32_t y) {
  const u32x2_t v = {x, y};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

// Interleaving of the per-channel key scale or zero inside a quad of lanes
// (all 4 active): lane k holds the fp16 pair of channels (2k, 2k+1) of the
// quad's 8 channels; the result of lane k is the pair (k, k + 4), the low
// halves of lanes 0 and 2 for k = 0, their high halves for k = 1, the low
// halves of lanes 1 and 3 for k = 2 and their high halves for k = 3.
__device__ __forceinline__ uint32_t quad_interleave(uint32_t x, int lane) {
  const uint32_t a = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x50, 0xF, 0xF, false));  // [0,0,1,1]
  const uint32_t b = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0xFA, 0xF, 0xF, false));  // [2,2,3,3]
  // (low of a, low of b) or (high of a, high of b)
  return __builtin_amdgcn_perm(b, a, (lane & 1) ? 0x07060302u : 0x05040100u);
}

// fp16 bit pattern of a binary32 value, nearest-even; zero is stored as +0.
__device__ __forceinline__ uint16_t f16_bits_canon(float f) {
  return f == 0.0f ? uint16_t(0) : __half_as_ushort(__float2half_rn(f));
}

// Per-group constants: minimum, binary32 scale s = (max - min) / qmax (IEEE
// division) and the reciprocal used by the fast path, v_rcp_f32 (within 1 ulp
// of 1/s; the fast-path bound below allows 4 ulp).  rcp = 0 when s == 0
// (every code is then 0).  Returns true when s is so small that 1/s could
// leave the normal range; rcp is then 0 and the block's codes must take the
// exact division.  Only bf16 inputs can get there: the smallest nonzero fp16
// scale is 2^-24 / 15.
template <int QMAX>
__device__ __forceinline__ bool group_consts(float mn, float mx, float& s, float& rcp) {
#pragma clang fp contract(off)
  s = (mx - mn) / static_cast<float>(QMAX);
  const bool tiny = s != 0.0f && s < 0x1p-100f;
  rcp = (s == 0.0f || tiny) ? 0.0f : __builtin_amdgcn_rcpf(s);
  return tiny;
}

// Code of x: rne(RN(RN(x - mn) / s)).  The clamp to [0, qmax] of the
// definition never changes a code here: 0 <= RN(x - mn) <= RN(mx - mn) and
// s = RN(RN(mx - mn) / qmax), so RN(RN(x - mn) / s) <= qmax * (1 + 2^-23),
// which rounds to at most qmax.
//
// Fast path y = RN(d * rcp).  With rcp = (1/s)(1 + e), |e| <= 4 * 2^-24, and
// d / s <= 16: |y - d / s| <= 16 * (2^-22 + 2^-24 + 2^-46) < 1.25 * 2^-18 and
// |RN(d / s) - d / s| <= 16 * 2^-24 = 0.25 * 2^-18, so y is within 1.5 * 2^-18
// of RN(d / s).  Rounding y to an integer therefore gives the same result
// unless y lies within 2^-17 of a half-integer.
//
// Near ties are repaired in one of two ways (Tie::kMask for bf16 inputs with
// 32-token blocks, whose coarse grid makes ties about ten times as frequent,
// Tie::kDev otherwise; with 64-token blocks the mask's registers would cost
// more resident workgroups than the repair saves):
//   kDev:  the fast pass only keeps the largest |y - rint(y)| of the thread
//          (one v_max per code).  A thread above 0.5 - 2^-17 runs the careful
//          pass: the same loop, in which the codes near a tie take the IEEE
//          division of the definition.  Cheapest in registers.
//   kMask: the fast pass sets the bit of every code near a tie in a per-thread
//          mask; only those codes are recomputed by the definition and patched
//          into their words (key_fix, value_fix).  Cheapest when most waves
//          hold a tie (bf16 with 4-bit codes: 98% of the waves), at the price
//          of more registers (fewer resident workgroups).
// A block with a tiny scale runs the careful pass (every code divides).
constexpr float kTieMargin = 0.49999237060546875f;  // 0.5 - 2^-17
enum class Tie { kDev, kMask, kCareful };
// one bit per code of a thread: G codes
template <int G>
using TieMask = typename std::conditional<G == 32, uint32_t, uint64_t>::type;
// per-thread tie state of the fast pass: the largest deviation, or the mask
template <Tie T, int G>
using TieState = typename std::conditional<T == Tie::kMask, TieMask<G>, float>::type;
template <Tie T, typename M>
__device__ __forceinline__ float code_of(float d, float rcp, float s, bool tiny, M& st, M bit) {
#pragma clang fp contract(off)
  const float y = d * rcp;
  float r = rintf(y);
  if constexpr (T == Tie::kCareful) {
    if (tiny || !(fabsf(y - r) <= kTieMargin)) r = s == 0.0f ? 0.0f : rintf(d / s);
  } else if constexpr (T == Tie::kMask) {
    if (!(fabsf(y - r) <= kTieMargin)) st |= bit;
  } else {
    st = fmaxf(st, fabsf(y - r));
  }
  return r;
}

// The code of element x of a group (minimum mn, scale s) by the definition:
// rne(RN(RN(x - mn) / s)), 0 when s == 0.
template <bool BF16>
__device__ __forceinline__ uint32_t exact_code(uint16_t xb, float mn, float s) {
#pragma clang fp contract(off)
  const float x = BF16 ? __uint_as_float(static_cast<uint32_t>(xb) << 16) : __half2float(__ushort_as_half(xb));
  return s == 0.0f ? 0u : static_cast<uint32_t>(rintf((x - mn) / s));
}

// d = RN(x - mn) for element SEL (0: low, 1: high half) of a packed pair.
// fp16: one v_fma_mix_f32 computes x * 1 - mn with a single rounding (the
// fp16 operand is widened exactly), i.e. the same RN(x - mn).
template <bool BF16, int SEL>
__device__ __forceinline__ float diff(uint32_t pair, float mn) {
#pragma clang fp contract(off)
  if constexpr (BF16) {
    const float x = SEL ? __uint_as_float(pair & 0xffff0000u) : __uint_as_float(pair << 16);
    return x - mn;
  } else {
    float d;
    if constexpr (SEL == 0) {
      asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(pair), "v"(mn));
    } else {
      asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(pair), "v"(mn));
    }
    return d;
  }
}

// Codes are accumulated as exact binary32 integers: the even codes of a word
// (its low half) as sum c * 2^(b*k) and the odd codes likewise; each half
// stays below 2^16, so every fma is exact.
__device__ __forceinline__ uint32_t halves_to_word(float lo, float hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

__device__ __forceinline__ float lo_f16(uint32_t w) { return __half2float(__ushort_as_half(static_cast<uint16_t>(w))); }
__device__ __forceinline__ float hi_f16(uint32_t w) { return __half2float(__ushort_as_half(static_cast<uint16_t>(w >> 16))); }

// Minimum and maximum without the NaN quieting the compiler inserts before
// each IEEE min/max (inputs are finite, so the plain instructions give the
// same results): packed fp16 pairs, and three binary32 values.
__device__ __forceinline__ uint32_t pk_min_f16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t pk_max_f16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float min3_f32(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Largest value over the 64 lanes of the wave.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off)));
  return x;
}

// Orders this workgroup's LDS traffic; unlike __syncthreads it does not wait
// for the scale/zero stores just issued to complete.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Key code words of one thread: word w (channels w*PK .. w*PK+PK-1) of
// tokens tg, tg + TS, ...; the channels are taken 8 at a time (fewer live
// registers).  kt: the staged key tile; kmn, krc, ksc: per channel minimum,
// reciprocal and scale.
template <int KB, int G, bool BF16, Tie T>
__device__ __forceinline__ void key_words(const uint16_t* kt, const float* kmn, const float* krc,
                                          const float* ksc, int w, int tg, bool tiny,
                                          uint32_t* word, TieState<T, G>& st) {
#pragma clang fp contract(off)
  constexpr int PK = 32 / KB, KW = D / PK, TS = 128 / KW, NT = G / TS;
  float wlo[NT], whi[NT];  // the word's even / odd codes as exact integers
#pragma unroll
  for (int j = 0; j < NT; ++j) wlo[j] = whi[j] = 0.0f;
#pragma unroll 1
  for (int c8 = 0; c8 < PK; c8 += 8) {
    const int d0 = w * PK + c8;
    float mn[8], rc[8], sc[8];
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
      const float4 a4 = *reinterpret_cast<const float4*>(&kmn[d0 + i]);
      const float4 c4 = *reinterpret_cast<const float4*>(&krc[d0 + i]);
      mn[i] = a4.x; mn[i + 1] = a4.y; mn[i + 2] = a4.z; mn[i + 3] = a4.w;
      rc[i] = c4.x; rc[i + 1] = c4.y; rc[i + 2] = c4.z; rc[i + 3] = c4.w;
      if constexpr (T == Tie::kCareful) {
        const float4 s4 = *reinterpret_cast<const float4*>(&ksc[d0 + i]);
        sc[i] = s4.x; sc[i + 1] = s4.y; sc[i + 2] = s4.z; sc[i + 3] = s4.w;
      } else {
        sc[i] = sc[i + 1] = sc[i + 2] = sc[i + 3] = 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(&kt[(tg + j * TS) * RS + d0]);
      const uint32_t xw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        // codes c8 + i (even: low half) and c8 + i + 1 (odd: high half),
        // both at bit KB * (c8 + i) / 2 of their half
        // (mask bit of code n of token slot j: j * PK + n)
        const float wt = static_cast<float>(1 << (KB * ((c8 + i) >> 1)));
        const TieState<T, G> bit = T == Tie::kMask ? TieState<T, G>(TieMask<G>(1) << (j * PK + c8 + i)) : 0;
        wlo[j] = fmaf(code_of<T>(diff<BF16, 0>(xw[i >> 1], mn[i]), rc[i], sc[i], tiny, st, bit), wt, wlo[j]);
        whi[j] = fmaf(code_of<T>(diff<BF16, 1>(xw[i >> 1], mn[i + 1]), rc[i + 1], sc[i + 1], tiny, st,
                                 T == Tie::kMask ? TieState<T, G>(TieMask<G>(bit) << 1) : bit),
                      wt, whi[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) word[j] = halves_to_word(wlo[j], whi[j]);
}

// Value code words of one thread: channels d0, d0 + 1 (one channel group) and
// rows (G/2)*h .. (G/2)*h + G/2 - 1, taken 8 rows at a time.  vt: the staged
// value tile; vmn, vrc, vsc: per (group, row) minimum, reciprocal and scale.
template <int VB, int G, bool BF16, Tie T>
__device__ __forceinline__ void value_words(const uint16_t* vt, const float* vmn, const float* vrc,
                                            const float* vsc, int d0, int h, bool tiny,
                                            uint32_t* w0, uint32_t* w1, TieState<T, G>& st) {
#pragma clang fp contract(off)
  constexpr int PV = 32 / VB, HR = G / 2, NW = HR / PV;
  const int m = d0 / G;
  float l0[NW], h0[NW], l1[NW], h1[NW];  // even / odd codes of channels d0, d0+1
#pragma unroll
  for (int k = 0; k < NW; ++k) l0[k] = h0[k] = l1[k] = h1[k] = 0.0f;
#pragma unroll
  for (int r8 = 0; r8 < HR; r8 += 8) {
    const int sbase = m * G + HR * h + r8;
    float mn[8], rc[8], sc[8];
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
      const float4 a4 = *reinterpret_cast<const float4*>(&vmn[sbase + j]);
      const float4 c4 = *reinterpret_cast<const float4*>(&vrc[sbase + j]);
      mn[j] = a4.x; mn[j + 1] = a4.y; mn[j + 2] = a4.z; mn[j + 3] = a4.w;
      rc[j] = c4.x; rc[j + 1] = c4.y; rc[j + 2] = c4.z; rc[j + 3] = c4.w;
      if constexpr (T == Tie::kCareful) {
        const float4 s4 = *reinterpret_cast<const float4*>(&vsc[sbase + j]);
        sc[j] = s4.x; sc[j + 1] = s4.y; sc[j + 2] = s4.z; sc[j + 3] = s4.w;
      } else {
        sc[j] = sc[j + 1] = sc[j + 2] = sc[j + 3] = 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = r8 + j;  // row HR*h + r: word r / PV, position r % PV
      const uint32_t xw = *reinterpret_cast<const uint32_t*>(&vt[(HR * h + r) * RS + d0]);
      const int k = r / PV, pos = r % PV;
      const float wt = static_cast<float>(1 << (VB * (pos >> 1)));
      // (mask bits of row r: 2 r for channel d0, 2 r + 1 for channel d0 + 1)
      const TieState<T, G> bit = T == Tie::kMask ? TieState<T, G>(TieMask<G>(1) << (2 * r)) : 0;
      const float c0 = code_of<T>(diff<BF16, 0>(xw, mn[j]), rc[j], sc[j], tiny, st, bit);
      const float c1 = code_of<T>(diff<BF16, 1>(xw, mn[j]), rc[j], sc[j], tiny, st,
                                  T == Tie::kMask ? TieState<T, G>(TieMask<G>(bit) << 1) : bit);
      if (pos & 1) {
        h0[k] = fmaf(c0, wt, h0[k]);
        h1[k] = fmaf(c1, wt, h1[k]);
      } else {
        l0[k] = fmaf(c0, wt, l0[k]);
        l1[k] = fmaf(c1, wt, l1[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    w0[k] = halves_to_word(l0[k], h0[k]);
    w1[k] = halves_to_word(l1[k], h1[k]);
  }
}

// Recomputes the key codes flagged in `mask` (bit j * PK + n: code n of the
// word of token slot j) by the definition and patches them into `word`.
template <int KB, int G, bool BF16>
__device__ __forceinline__ void key_fix(const uint16_t* kt, const float* kmn, const float* ksc, int w, int tg,
                                     TieMask<G> mask, uint32_t* word) {
#pragma clang fp contract(off)
  constexpr int PK = 32 / KB, KW = D / PK, TS = 128 / KW, NT = G / TS;
  while (mask) {
    const int bit = __builtin_ctzll(static_cast<uint64_t>(mask));
    mask &= mask - 1;
    const int j = bit / PK, n = bit % PK, d = w * PK + n;
    const uint32_t c = exact_code<BF16>(kt[(tg + j * TS) * RS + d], kmn[d], ksc[d]);
    const int pos = KB * (n >> 1) + 16 * (n & 1);
    const uint32_t keep = ~(((1u << KB) - 1u) << pos);
#pragma unroll
    for (int jj = 0; jj < NT; ++jj)
      if (jj == j) word[jj] = (word[jj] & keep) | (c << pos);
  }
}

// Recomputes the value codes flagged in `mask` (bit 2 r + e: row r of the
// thread's rows, channel d0 + e) and patches them into w0 / w1.
template <int VB, int G, bool BF16>
__device__ __forceinline__ void value_fix(const uint16_t* vt, const float* vmn, const float* vsc, int d0, int h,
                                       TieMask<G> mask, uint32_t* w0, uint32_t* w1) {
#pragma clang fp contract(off)
  constexpr int PV = 32 / VB, HR = G / 2, NW = HR / PV;
  const int m = d0 / G;
  while (mask) {
    const int bit = __builtin_ctzll(static_cast<uint64_t>(mask));
    mask &= mask - 1;
    const int r = bit >> 1, e = bit & 1;
    const int gi = m * G + HR * h + r;  // the row's group constants
    const uint32_t c = exact_code<BF16>(vt[(HR * h + r) * RS + d0 + e], vmn[gi], vsc[gi]);
    const int k = r / PV, p = r % PV;
    const int pos = VB * (p >> 1) + 16 * (p & 1);
    const uint32_t keep = ~(((1u << VB) - 1u) << pos);
#pragma unroll
    for (int kk = 0; kk < NW; ++kk) {
      if (kk == k && e == 0) w0[kk] = (w0[kk] & keep) | (c << pos);
      if (kk == k && e == 1) w1[kk] = (w1[kk] & keep) | (c << pos);
    }
  }
}


// LDS of one block: the G x D key and value tiles (rows padded to RS
// elements) and the per-group minimum, scale and reciprocal of keys (per
// channel) and values (per channel group and row).
template <int G>
struct PackLds {
  static constexpr int kTile = G * RS * 2;  // bytes of one tile
  static constexpr int bytes = 2 * kTile + 6 * D * 4;
  uint16_t* kt;
  uint16_t* vt;
  float *kmn, *ksc, *krc, *vmn, *vsc, *vrc;
  __device__ explicit PackLds(uint8_t* base)
      : kt(reinterpret_cast<uint16_t*>(base)),
        vt(reinterpret_cast<uint16_t*>(base + kTile)),
        kmn(reinterpret_cast<float*>(base + 2 * kTile)),
        ksc(kmn + D), krc(ksc + D), vmn(krc + D), vsc(vmn + D), vrc(vsc + D) {}
};

// Packs one block: G tokens of keys and values (rows of D elements at ksrc
// and vsrc) into the block record `rec` (layout block_layout(KB, VB, G)) and
// writes the record's largest key and value scale to *smax_out.  NT threads
// (tid = 0 .. NT - 1, NT = 128 or 256, whole waves) take the work of 256 in
// turns; every phase hands whole waves the same role, so the wave
// reductions and barriers stay uniform.  All NT threads must call it; it
// ends with a barrier after its last LDS access, and its global stores may
// still be in flight.
template <int KB, int VB, bool BF16, int G, Tie TF, int NT>
__device__ __forceinline__ void pack_block(const uint16_t* __restrict__ ksrc, const uint16_t* __restrict__ vsrc,
                                           uint8_t* rec, uint32_t* smax_out, uint8_t* lds_base, int tid) {
#pragma clang fp contract(off)
  static_assert(NT == 128 || NT == 256, "whole waves");
  constexpr int QK = (1 << KB) - 1, QV = (1 << VB) - 1;
  constexpr int PK = 32 / KB;  // key codes (channels) per word
  constexpr int KW = D / PK;   // key words per token
  constexpr int PV = 32 / VB;  // value codes (rows) per word
  constexpr BlockLayout BL = block_layout(KB, VB, G);
  const PackLds<G> L(lds_base);
  uint16_t* const kt = L.kt;
  uint16_t* const vt = L.vt;
  float* const kmn = L.kmn;
  float* const ksc = L.ksc;
  float* const krc = L.krc;
  float* const vmn = L.vmn;
  float* const vsc = L.vsc;
  float* const vrc = L.vrc;
  // set when some group of the block has a scale below 2^-100; kept in the
  // padding of the first key row, next to the largest stored key and value
  // scale of the block (fp16 bit patterns: scales are >= 0, so their bit
  // patterns order like their values)
  int& tiny_scale = *reinterpret_cast<int*>(&kt[D]);
  uint32_t& smax_k = *reinterpret_cast<uint32_t*>(&kt[D + 2]);
  uint32_t& smax_v = *reinterpret_cast<uint32_t*>(&kt[D + 4]);

  {
    // ---- stage the key and value tiles: 16-byte pieces tid, tid + NT, ...
    // of the G x 128 tiles, all loads issued before the first LDS store
    constexpr int NP = G * (D / 8) / NT;
    uint4 kx[NP], vx[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int piece = tid + i * NT;
      const int off = (piece / (D / 8)) * D + (piece % (D / 8)) * 8;
      kx[i] = load_stream16(ksrc + off);
      vx[i] = load_stream16(vsrc + off);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int piece = tid + i * NT;
      const int off = (piece / (D / 8)) * RS + (piece % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&kt[off]) = kx[i];
      *reinterpret_cast<uint4*>(&vt[off]) = vx[i];
    }
    if (tid == 0) {
      tiny_scale = 0;
      smax_k = smax_v = 0u;
    }
  }
  __syncthreads();

  // ---- group statistics (min/max are exact in the input format; fp16
  // pairs use the packed min/max instructions).  Items 0 .. 63: key channel
  // pairs; 64 .. 191: value groups (whole waves).
#pragma unroll
  for (int it = tid; it < 256; it += NT) {
    if (it < D / 2) {
      // key groups: channels 2p, 2p+1 over the G rows of the block
      const int p2 = 2 * it;
      float mn0, mx0, mn1, mx1;
      if constexpr (BF16) {
        uint32_t x = *reinterpret_cast<const uint32_t*>(&kt[p2]);
        mn0 = mx0 = __uint_as_float(x << 16);
        mn1 = mx1 = __uint_as_float(x & 0xffff0000u);
#pragma unroll 4
        for (int t = 1; t < G; t += 2) {
          const uint32_t x0 = *reinterpret_cast<const uint32_t*>(&kt[t * RS + p2]);
          const uint32_t x1 = t + 1 < G ? *reinterpret_cast<const uint32_t*>(&kt[(t + 1) * RS + p2]) : x0;
          const float l0 = __uint_as_float(x0 << 16), h0 = __uint_as_float(x0 & 0xffff0000u);
          const float l1 = __uint_as_float(x1 << 16), h1 = __uint_as_float(x1 & 0xffff0000u);
          mn0 = min3_f32(mn0, l0, l1); mx0 = max3_f32(mx0, l0, l1);
          mn1 = min3_f32(mn1, h0, h1); mx1 = max3_f32(mx1, h0, h1);
        }
      } else {
        uint32_t mn = *reinterpret_cast<const uint32_t*>(&kt[p2]), mx = mn;
#pragma unroll 8
        for (int t = 1; t < G; ++t) {
          const uint32_t x = *reinterpret_cast<const uint32_t*>(&kt[t * RS + p2]);
          mn = pk_min_f16(mn, x);
          mx = pk_max_f16(mx, x);
        }
        mn0 = lo_f16(mn); mn1 = hi_f16(mn);
        mx0 = lo_f16(mx); mx1 = hi_f16(mx);
      }
      float s0, r0, s1, r1;
      const bool t0 = group_consts<QK>(mn0, mx0, s0, r0);
      const bool t1 = group_consts<QK>(mn1, mx1, s1, r1);
      if (t0 || t1) tiny_scale = 1;
      kmn[p2] = mn0; ksc[p2] = s0; krc[p2] = r0;
      kmn[p2 + 1] = mn1; ksc[p2 + 1] = s1; krc[p2 + 1] = r1;
      const uint32_t sb0 = f16_bits_canon(s0), sb1 = f16_bits_canon(s1);
      const uint32_t top = wave_max(max(sb0, sb1));  // one wave: all 128 key channels
      if ((it & 63) == 0) atomicMax(&smax_k, top);
      // stored interleaved: word w of each 8 channels holds channels w and
      // w + 4 (the pairing of the decode's code conversions).  Lane k of a
      // quad holds channels 2k, 2k+1 of the quad's 8; word k takes the low
      // (k even) or high (k odd) halves of lanes k / 2 and k / 2 + 2.
      const uint32_t zb = f16_bits_canon(mn0) | (static_cast<uint32_t>(f16_bits_canon(mn1)) << 16);
      store_stream(reinterpret_cast<uint32_t*>(rec + BL.k_scale) + it, quad_interleave(sb0 | (sb1 << 16), it));
      store_stream(reinterpret_cast<uint32_t*>(rec + BL.k_zero) + it, quad_interleave(zb, it));
    } else if (it < D / 2 + D) {
      // value group: row t, channels m*G .. m*G+G-1; index i = m*G + t
      const int i = it - D / 2;
      const int m = i / G, t = i % G;
      const uint4* row = reinterpret_cast<const uint4*>(&vt[t * RS + m * G]);
      float mn, mx;
      if constexpr (BF16) {
        mn = INFINITY;
        mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < G / 8; ++c) {
          const uint4 v = row[c];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float lo = __uint_as_float(w4[j] << 16), hi = __uint_as_float(w4[j] & 0xffff0000u);
            mn = min3_f32(mn, lo, hi);
            mx = max3_f32(mx, lo, hi);
          }
        }
      } else {
        uint32_t pmn = 0, pmx = 0;
#pragma unroll
        for (int c = 0; c < G / 8; ++c) {
          const uint4 v = row[c];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pmn = (c == 0 && j == 0) ? w4[j] : pk_min_f16(pmn, w4[j]);
            pmx = (c == 0 && j == 0) ? w4[j] : pk_max_f16(pmx, w4[j]);
          }
        }
        // fp16 -> binary32 is exact and order preserving
        mn = fminf(lo_f16(pmn), hi_f16(pmn));
        mx = fmaxf(lo_f16(pmx), hi_f16(pmx));
      }
      float s, rcp;
      if (group_consts<QV>(mn, mx, s, rcp)) tiny_scale = 1;
      vmn[i] = mn;
      vsc[i] = s;
      vrc[i] = rcp;
      const uint32_t sb = f16_bits_canon(s);
      const uint32_t top = wave_max(sb);  // two waves: 64 value groups each
      if ((it & 63) == 0) atomicMax(&smax_v, top);
      store_stream(reinterpret_cast<uint16_t*>(rec + BL.v_scale) + i, static_cast<uint16_t>(sb));  // [m][row]
      store_stream(reinterpret_cast<uint16_t*>(rec + BL.v_zero) + i, f16_bits_canon(mn));
    }
  }
  lds_barrier();

  // the record's largest key and value scale, for the decode's operand range
  if (tid == 0) store_stream(smax_out, smax_k | (smax_v << 16));
  const bool tiny = tiny_scale != 0;
#pragma unroll
  for (int it = tid; it < 256; it += NT) {
    if (it < 128) {
      // ---- key code words: word w of token t holds channels w*PK .. w*PK+PK-1.
      // Item: one word index w, tokens tg, tg + TS, ... (NT tokens).
      constexpr int TS = 128 / KW, NTK = G / TS;
      const int w = it % KW, tg = it / KW;
      uint32_t word[NTK];
      TieState<TF, G> st = 0;
      key_words<KB, G, BF16, TF>(kt, kmn, krc, ksc, w, tg, false, word, st);
      float no_state = 0.0f;  // the careful pass keeps no tie state
      if (tiny || (TF == Tie::kDev && st > kTieMargin)) {
        asm volatile("" ::: "memory");  // reload the tile: nothing kept live across the passes
        key_words<KB, G, BF16, Tie::kCareful>(kt, kmn, krc, ksc, w, tg, tiny, word, no_state);
      } else if constexpr (TF == Tie::kMask) {
        if (st) key_fix<KB, G, BF16>(kt, kmn, ksc, w, tg, st, word);
      }
      uint32_t* const kc = reinterpret_cast<uint32_t*>(rec + BL.k_codes);
#pragma unroll
      for (int j = 0; j < NTK; ++j) store_stream(kc + (tg + j * TS) * KW + w, word[j]);
    } else {
      // ---- value code words: word w of channel d holds rows w*PV .. w*PV+PV-1;
      // word-major, the D words of one w adjacent.  Item: channels d0, d0+1
      // (same channel group) and rows (G/2)*h .. (G/2)*h + G/2 - 1.
      const int i0 = it - 128;
      const int d0 = 2 * (i0 % 64), h = i0 / 64;
      constexpr int NW = (G / 2) / PV;
      uint32_t w0[NW], w1[NW];
      TieState<TF, G> st = 0;
      value_words<VB, G, BF16, TF>(vt, vmn, vrc, vsc, d0, h, false, w0, w1, st);
      float no_state = 0.0f;  // the careful pass keeps no tie state
      if (tiny || (TF == Tie::kDev && st > kTieMargin)) {
        asm volatile("" ::: "memory");  // reload the tile: nothing kept live across the passes
        value_words<VB, G, BF16, Tie::kCareful>(vt, vmn, vrc, vsc, d0, h, tiny, w0, w1, no_state);
      } else if constexpr (TF == Tie::kMask) {
        if (st) value_fix<VB, G, BF16>(vt, vmn, vsc, d0, h, st, w0, w1);
      }
      uint32_t* const vc = reinterpret_cast<uint32_t*>(rec + BL.v_codes);
#pragma unroll
      for (int k = 0; k < NW; ++k)
        store_stream2(&vc[(h * NW + k) * D + d0], w0[k], w1[k]);
    }
  }
  __syncthreads();  // the tile may be reused
}

}  // namespace packcore
}  // namespace kivi
