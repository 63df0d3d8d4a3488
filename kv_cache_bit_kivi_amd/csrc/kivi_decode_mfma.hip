// kivi_decode_mfma.hip - decode attention with both contractions on the
// matrix cores, for 1, 2, 4, 8 or 16 query heads per kv head (multi-head and
// grouped-query attention).  A workgroup serves up to 4 query heads in 4 head
// slots of the matrix columns (spare slots carry zeros and are masked out),
// or 8 in the eight-head layout (key_wave8, value_wave8); 16 heads take 2
// workgroups (head groups) per split, launched side by side on one XCD so
// that the second reads the records from its L2.
//
// Method: split-K decode attention over the packed cache (dequantized value =
// code * scale + zero, page "KIVI: Asymmetric 2-Bit KV Cache Quantization
// Guide", "Step 2"), fused with the dequantization as the pages require for
// the memory saving to turn into speed (page "KV-Cache Quantization: I Ran the
// Experiments", "Where it still breaks", item 3).
//
// One workgroup of two waves per (unit, split): a key wave computes scores
// and the online softmax, a value wave accumulates p.V one step behind it;
// they meet once per step at a workgroup barrier and hand over the
// probabilities through LDS.  The scales are folded into the dense operand
// of each product so that the codes themselves feed the matrix cores:
//   q . k^_t   = sum_d (q_d S_gd) c_td + sum_d q_d Z_gd         (key group g)
//   sum_t p_t v^_t,d = sum_t (p_t S_tm) c_td + sum_t p_t Z_tm   (value group m)
// Codes enter v_mfma_f32_16x16x32_f16 as the normal fp16 numbers c * 2^(F-15)
// (exact), extracted from the split-half words by two masks per word and one
// fp4/fp8 conversion per pair.  The folded operands q*S and p*S are carried
// as fp16 hi + lo pairs: q*S exactly, p*S within 2^-22 relative.  With 4 heads
// in a workgroup the pair takes two products; with 1 or 2 the lo halves ride
// in the spare head-slot columns of the same product.  The zero-point term of
// the keys (one dot product per group and head) runs on the vector ALUs.
//
// Key side: four consecutive 32-token groups at once, block-diagonal: A rows
// are 4 tokens of each of the 4 groups, B columns are the 4 heads x 4 groups,
// so each lane builds distinct q*S values; the 16 diagonal lanes hold the
// scores.  Value side, per group: A = codes of 16 channels x 32 tokens, B
// columns = 4 heads x 4 channel groups m (p*S differs per m); each output
// lane keeps the column of its own channel group.
//
// Softmax: the scores of a step pass through LDS so that each of the 64
// lanes exponentiates 8 of them (the matrix layout leaves them on 16 lanes).
//
// The residual window (at most R tokens, stored in kv dtype) is handled on the
// vector ALUs in fp32 by the value wave of the unit's last packed split, after
// its packed groups, as a partial of its own.
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int G = kGroup;
constexpr int D = kHeadDim;
constexpr int GQ = 4;  // head slots of a wave (matrix columns); NQ <= GQ are used
constexpr int kRowP = 36;  // LDS row of one (stream, head): 32 scores + 4 floats padding

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  } else {
    return __half2float(__ushort_as_half(h));
  }
}

__device__ __forceinline__ f32x4 mfma(const half8_t& a, const half8_t& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8_t as_h8(const u32x4& v) { return __builtin_bit_cast(half8_t, v); }

__device__ __forceinline__ float lo_half(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float hi_half(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Two binary32 values to an fp16 pair, each rounded to nearest-even (one
// v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pk_rne(float x0, float x1) {
  const half2_t h = {static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
  return __builtin_bit_cast(uint32_t, h);
}

// x - (fp16 half `sel` of h), one v_fma_mix_f32 (the half is read as fp16).
template <int SEL>
__device__ __forceinline__ float minus_half(uint32_t h, float x) {
  float r;
  if constexpr (SEL == 0) {
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  } else {
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  }
  return r;
}

// x * (fp16 half `sel` of h), one v_fma_mix_f32 (exact product, one rounding).
template <int SEL>
__device__ __forceinline__ float times_half(float x, uint32_t h) {
  float r;
  if constexpr (SEL == 0) {
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(h));
  } else {
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(h));
  }
  return r;
}

// (x0, x1) -> fp16 pairs hi (nearest) and lo (nearest of the exact remainder
// x - hi): hi + lo = x within 2^-22 relative.  |x| must stay below 65504.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pk_rne(x0, x1);
  lo = pk_rne(minus_half<0>(hi, x0), minus_half<1>(hi, x1));
}

// Exact product of two fp16 pairs as hi + lo fp16 pairs: hi = RN(a * b)
// (v_pk_mul_f16) and lo = RN(a * b - hi) (v_pk_fma_f16, one rounding of the
// exact value).  An fp16 product has at most 22 significant bits, so lo is
// the exact remainder unless it falls below the fp16 subnormal step 2^-24
// (an absolute error of at most 2^-25).  |a * b| must stay below 65504.
__device__ __forceinline__ void mul_pair_exact(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
  asm("v_pk_mul_f16 %0, %1, %2" : "=v"(hi) : "v"(a), "v"(b));
  asm("v_pk_fma_f16 %0, %1, %2, %3 neg_lo:[0,0,1] neg_hi:[0,0,1]" : "=v"(lo) : "v"(a), "v"(b), "v"(hi));
}

// RN(a * b - RN(m * b)) for fp16 pairs: with m = a the exact remainder of
// mul_pair_exact's hi (its lo), with m = 0 the hi itself.
__device__ __forceinline__ uint32_t residual_pair(uint32_t a, uint32_t b, uint32_t m) {
  uint32_t h, r;
  asm("v_pk_mul_f16 %0, %1, %2" : "=v"(h) : "v"(m), "v"(b));
  asm("v_pk_fma_f16 %0, %1, %2, %3 neg_lo:[0,0,1] neg_hi:[0,0,1]" : "=v"(r) : "v"(a), "v"(b), "v"(h));
  return r;
}

// acc + a.x * b.x + a.y * b.y for fp16 pairs a, b (v_dot2_f32_f16).
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), acc, false);
}

// Code extraction.  In a split-half word the codes of one byte sit at bit
// steps of b (the 4 codes of a 2-bit byte, the 2 codes of a 4-bit byte).
// Masking with 0x33333333 (2-bit; also after a shift by 2) leaves one 2-bit
// code in the low bits of each nibble, which as an fp4 e2m1 number is c / 2;
// masking with 0x0F0F0F0F (4-bit; also after a shift by 4) leaves one code per
// byte, which as an fp8 e4m3 number is c * 2^-9.  The gfx950 conversions
// v_cvt_scalef32_pk_f16_fp4 (two nibbles of a byte) and _fp8 (two bytes of a
// half word) turn them into two fp16 numbers times a power-of-two scale,
// exactly: every code becomes the normal fp16 number c * 2^(F-15) (F = 6 for
// 2-bit, 4 for 4-bit), zero stays zero.  A conversion pairs the codes of
// entries a and a + 4 of a run of 8 (a = 0..3), so the dense operand of
// every product takes the same pairing (the record stores the key scale and
// zero interleaved in that order; the value wave picks scale halves per
// token).
//
// Normal operands matter for the accuracy of the products: measured on
// MI355X, a v_mfma_f32_16x16x32_f16 whose A operand holds fp16 subnormals
// (codes masked in place, c * 2^(t-24) at bit position t, with position
// factors in the other operand) adds its products with errors of hundreds of
// binary32 units relative to the sum of their magnitudes (270 at 4 bits,
// 850-1260 at 2 bits, worst over 25600 sums of 128 products), while the same
// products from normal operands come within 5 units.  In attention those
// errors reached the 2e-3 tolerance where one token holds most of a head's
// weight and its value is large.
template <int BITS>
struct CodeScale {
  static constexpr int F = BITS == 2 ? 6 : 4;
};

// 8 codes (one run of 8 consecutive entries: positions 8*HB .. 8*HB+7 of
// word x; 4-bit words hold one run, HB = 0) as four fp16 pairs c * 2^(F-15):
// pair a holds entries a and a + 4 of the run.
template <int BITS, int HB>
__device__ __forceinline__ half8_t codes8(uint32_t x) {
  u32x4 r;
  if constexpr (BITS == 2) {
    // the nibbles of y0 hold entries (0, 4), (8, 12), (1, 5), (9, 13) by
    // byte, those of y1 entries (2, 6), (10, 14), (3, 7), (11, 15)
    const uint32_t y0 = x & 0x33333333u, y1 = (x >> 2) & 0x33333333u;
    constexpr float kScale = 0x1p-8f;  // c / 2 -> c * 2^-9
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, kScale, HB));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, kScale, 2 + HB));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, kScale, HB));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, kScale, 2 + HB));
  } else {
    static_assert(HB == 0, "a 4-bit word holds one run");
    // bytes of z0: entries 0, 4, 1, 5; of z1: 2, 6, 3, 7
    const uint32_t z0 = x & 0x0F0F0F0Fu, z1 = (x >> 4) & 0x0F0F0F0Fu;
    constexpr float kScale = 0x1p-2f;  // c * 2^-9 -> c * 2^-11
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(z0, kScale, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(z0, kScale, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(z1, kScale, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(z1, kScale, true));
  }
  return as_h8(r);
}

// Cross-lane exchanges on the vector ALUs (no LDS round trip):
//   lane ^ 1, lane ^ 2 : DPP quad permutations
//   lane ^ 16          : v_permlane16_swap (rows 0<->1, 2<->3)
//   lane ^ 32          : v_permlane32_swap (halves)
// Each returns the value of the partner lane combined with the own value.
template <int M>
__device__ __forceinline__ float partner(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  } else {
    static_assert(M == 16 || M == 32, "exchange");
    return 0.0f;
  }
}

// Reductions over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15): the
// quad exchanges (lane ^ 1, lane ^ 2) leave each lane its quad's result, the
// half-row mirror (lane i <-> 7 - i of each 8) combines the two quads of a
// half row and the row mirror (i <-> 15 - i) the two halves.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppHalfMirror = 0x141, kDppMirror = 0x140;

// max(a, b) as one v_max_f32: the operands are scores or -inf, never NaN, so
// the NaN quieting the compiler adds to fmaxf (one more instruction per
// operand that it cannot prove canonical, such as a cross-lane result) is
// not needed.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// reduce over lanes l ^ 16 / l ^ 32: after the swap the two results hold
// (own, partner) in some order on every lane, so op(r0, r1) is the pair op
template <int M>
__device__ __forceinline__ float swap_max(float v) {
  const uint32_t x = __float_as_uint(v);
  auto r = (M == 16) ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                     : __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int M>
__device__ __forceinline__ float swap_sum(float v) {
  const uint32_t x = __float_as_uint(v);
  auto r = (M == 16) ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                     : __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float row_max16(float v) {
  v = max_raw(v, partner<1>(v));
  v = max_raw(v, partner<2>(v));
  v = max_raw(v, dpp_f<kDppHalfMirror>(v));
  return max_raw(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v = v + partner<1>(v);
  v = v + partner<2>(v);
  v = v + dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}
__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }

// ---------------------------------------------------------------------------
// Synchronisation.  global->LDS loads are counted by vmcnt and complete in
// issue order; one wave's LDS operations execute in order, so waiting for
// this wave's own LDS operations (lgkmcnt) orders its LDS traffic without
// draining the loads still in flight.  (__syncthreads would wait for them.)

// Waits until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Keeps the compiler from moving LDS accesses across this point.  LDS
// operations of one wave execute in issue order, so LDS data written by some
// lanes is visible to reads issued after it by other lanes of the wave; the
// compiler, which reasons per lane, must not reorder such a read above the
// write.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// Both waves of the workgroup: this wave's LDS writes are complete, then
// meet.  Outstanding global->LDS loads stay in flight.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Parity of a step (which half of the double buffers it uses): a constant
// when the step loop runs in pairs, else from the step index.
struct RuntimeParity {};
template <int P>
__device__ __forceinline__ constexpr int parity(int, std::integral_constant<int, P>) { return P; }
__device__ __forceinline__ int parity(int step, RuntimeParity) { return step & 1; }

// Runs steps 0 .. n_steps - 1 of a wave.  In pairs (even and odd steps use
// fixed halves of the double buffers, so their LDS offsets are constants),
// except for 4-bit keys with 2-bit values, whose register budget the doubled
// loop body exceeds.
template <bool PAIRS, typename F>
__device__ __forceinline__ void run_steps(int n_steps, F&& one_step) {
  if constexpr (PAIRS) {
    for (int step = 0; step < n_steps; step += 2) {
      one_step(step, std::integral_constant<int, 0>{});
      if (step + 1 < n_steps) one_step(step + 1, std::integral_constant<int, 1>{});
    }
  } else {
    for (int step = 0; step < n_steps; ++step) one_step(step, RuntimeParity{});
  }
}

// ---------------------------------------------------------------------------
// Residual window on the vector ALUs (one wave, fp32), written as its own
// partial.  qsh / psh: LDS scratch of this wave.
template <bool BF16, int NQ>
__device__ void window_wave(const DecodeArgs& a, long long u, int b, int h0, int split, int nr,
                            bool store_token, float (*qsh)[D], float (*psh)[G]) {
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < NQ * D; i += 64) {
    qsh[i / D][i % D] =
        to_f32<BF16>(a.q[((long long)b * a.Hq + h0 + i / D) * D + i % D]) * a.qscale;
  }
  // fused append: the newest token (slot nr - 1) comes from k_new / v_new;
  // this wave (of the unit's first head group) is the only one of the launch
  // that writes the unit's window, so it also stores the token there
  const int t_new = a.k_new ? nr - 1 : -1;
  if (t_new >= 0 && store_token) {
    const long long src = u * D + 2 * lane, dst = (u * a.R + t_new) * D + 2 * lane;
    *reinterpret_cast<uint32_t*>(a.k_resid_w + dst) = *reinterpret_cast<const uint32_t*>(a.k_new + src);
    *reinterpret_cast<uint32_t*>(a.v_resid_w + dst) = *reinterpret_cast<const uint32_t*>(a.v_new + src);
  }
  wave_lds_sync();
  float m[NQ], l[NQ], o[NQ][2];
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
    o[h][0] = o[h][1] = 0.0f;
  }
  const int half = lane >> 5;
  for (int c0 = 0; c0 < nr; c0 += G) {
    const int t = c0 + (lane & 31);
    const bool live = t < nr;
    float acc[NQ];
#pragma unroll
    for (int h = 0; h < NQ; ++h) acc[h] = 0.0f;
    if (live) {
      const uint16_t* kr = (t == t_new ? a.k_new + u * D : a.k_resid + (u * a.R + t) * D) + 64 * half;
      for (int d0 = 0; d0 < 64; d0 += 8) {
        const uint4 kv = *reinterpret_cast<const uint4*>(kr + d0);
        const uint32_t ww[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float kx = to_f32<BF16>(static_cast<uint16_t>(ww[i >> 1] >> (16 * (i & 1))));
#pragma unroll
          for (int h = 0; h < NQ; ++h) acc[h] = fmaf(qsh[h][64 * half + d0 + i], kx, acc[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      float s = acc[h] + __shfl_xor(acc[h], 32);
      s = live ? s : -INFINITY;
      float mx = s;
      for (int off = 16; off > 0; off >>= 1) mx = xor_max(mx, off);
      const float m_new = fmaxf(m[h], mx);
      const float alpha = (m[h] == -INFINITY) ? 0.0f : exp2f(m[h] - m_new);
      const float p = live ? exp2f(s - m_new) : 0.0f;
      float ps = p;
      for (int off = 16; off > 0; off >>= 1) ps = xor_sum(ps, off);
      l[h] = l[h] * alpha + ps;
      m[h] = m_new;
      o[h][0] *= alpha;
      o[h][1] *= alpha;
      if (lane < G) psh[h][lane] = p;
    }
    wave_lds_sync();
    const int n = min(G, nr - c0);
    for (int tt = 0; tt < n; ++tt) {
      const uint16_t* vr = c0 + tt == t_new ? a.v_new + u * D : a.v_resid + (u * a.R + c0 + tt) * D;
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(vr + 2 * lane);
      const float v0 = to_f32<BF16>(static_cast<uint16_t>(vv & 0xffffu));
      const float v1 = to_f32<BF16>(static_cast<uint16_t>(vv >> 16));
#pragma unroll
      for (int h = 0; h < NQ; ++h) {
        o[h][0] = fmaf(psh[h][tt], v0, o[h][0]);
        o[h][1] = fmaf(psh[h][tt], v1, o[h][1]);
      }
    }
    wave_lds_sync();
  }
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    float* P = a.partial + (((long long)b * a.Hq + h0 + h) * a.n_split + split) * (D + 2);
    P[2 + 2 * lane] = o[h][0];
    P[3 + 2 * lane] = o[h][1];
    if (lane == 0) {
      P[0] = m[h];
      P[1] = l[h];
    }
  }
}

// ---------------------------------------------------------------------------
// LDS of one workgroup.  A step covers 4 consecutive packed groups of one
// unit; stages are filled by direct global->LDS loads (64 lanes x 16 bytes =
// 1 KiB per instruction).
//   key codes   x1 (key wave): 4 groups x 32 rows x D*KB/8 bytes, each group
//               padded by 64 bytes (the 4 groups fall on different banks);
//               refilled with the next step's codes as soon as this step's
//               are in registers
//   key meta    x2: scale 4 x D fp16, zero 4 x D fp16
//   value stage x2 (value wave): codes 4 groups x (G/PV words) x D words;
//               scale 4 x 4 x G fp16; zero likewise.
//   hand-over   x2: scores, then in place probabilities [stream][head][kRowP]
//               fp32, and the rescale factor of each head, written by the key
//               wave.
// NH: query heads of a workgroup (4, or 8 in the eight-head layout).
template <int KB, int VB, int NH = GQ>
struct Stage {
  static constexpr int kRow = D * KB / 8;              // bytes per key row
  static constexpr int kGroup = G * kRow;              // 1 or 2 KiB
  static constexpr int kGroupPad = kGroup + 64;
  static constexpr int kCodeBytes = 4 * kGroupPad;
  static constexpr int kMetaBytes = 2 * 4 * D * 2;       // scale, then zero
  static constexpr int offKM0 = kCodeBytes;
  static constexpr int vGroup = (G * VB / 32) * D * 4; // 1 or 2 KiB
  static constexpr int offVS = 4 * vGroup, offVZ = offVS + 4 * D * 2;
  static constexpr int vBytes = offVZ + 4 * D * 2;
  static constexpr int offAlpha = 4 * NH * kRowP * 4;   // in a hand-over buffer
  static constexpr int offBias = offAlpha + 4 * NH;      // zero-point terms [stream][head]
  static constexpr int pBytes = offBias + 4 * NH * 4;
  static constexpr int offV0 = offKM0 + 2 * kMetaBytes, offP0 = offV0 + 2 * vBytes;
  static constexpr int bytes = offP0 + 2 * pBytes;     // LDS per workgroup
  static constexpr int kLoads = (4 * kGroup + 2 * 4 * D * 2) / 1024;  // DMA instructions
  static constexpr int vLoads = (4 * vGroup + 2 * 4 * D * 2) / 1024;
  static_assert(vBytes >= (NH * D + NH * G) * 4, "window scratch fits in a value stage");
};
static_assert(Stage<2, 2>::bytes == mfma_wg_lds_bytes(2, 2, 4), "lds");
static_assert(Stage<4, 4>::bytes == mfma_wg_lds_bytes(4, 4, 4), "lds");
static_assert(Stage<2, 4>::bytes == mfma_wg_lds_bytes(2, 4, 4), "lds");
static_assert(Stage<4, 2>::bytes == mfma_wg_lds_bytes(4, 2, 4), "lds");
static_assert(Stage<2, 2, 8>::bytes == mfma_wg_lds_bytes(2, 2, 8), "lds");
static_assert(Stage<4, 4, 8>::bytes == mfma_wg_lds_bytes(4, 4, 8), "lds");
static_assert(Stage<2, 4, 8>::bytes == mfma_wg_lds_bytes(2, 4, 8), "lds");
static_assert(Stage<4, 2, 8>::bytes == mfma_wg_lds_bytes(4, 2, 8), "lds");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef const __attribute__((address_space(1))) void glb_void_t;

// 16 bytes per lane from global memory to LDS.  Records are read once, with
// the streaming hint (nt), unless several head groups read them (KEEP): the
// other workgroups of the pair then find them in the XCD's L2.  (The hint is
// an immediate of the instruction, hence a template argument: a run-time
// flag costs a branch around every load.)
template <bool KEEP>
__device__ __forceinline__ void dma16(const void* src, lds_u8* lds_dst) {
  // address-space conversions need C-style casts
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_dst, 16, 0, KEEP ? 0 : 2);
}

// 16 bytes per lane from a step's records to LDS through a buffer resource
// (unit-major caches): byte offset voff (per lane) + soff (uniform) from the
// step's first record; the resource's size bounds every access.  Streaming
// hint as in dma16.
template <bool KEEP>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff, lds_u8* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_dst, 16, voff, soff, 0, KEEP ? 0 : 2);
}

// Buffer resource over the records of the 4 streams of a step starting at
// stream g0 of a unit-major unit (at most 4 records from the record of g0;
// gfx9 raw buffer: stride 0, size in bytes, default data format word).  The
// 64-bit base keeps the 32-bit offsets small for a unit of any size.
template <int GT, int BYTES>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t step_rsrc(const uint8_t* ubase, int g0) {
  const uint8_t* base = ubase + static_cast<size_t>(g0 / (GT / kStream)) * BYTES;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0), 4 * BYTES, 0x00020000);
}

// Records of streams g0 .. g0 + 3 of unit u (unit-major, or through the
// page table when PAGED).  A stream is 32 tokens: a whole block of G = 32, or
// half `hf` of a block of G = 64.  Slots past the last valid stream
// g0 + ns - 1 repeat it (addresses stay inside).  ubase: the unit's first
// record (unit-major); the step's records then lie a few records apart.
template <int KB, int VB, int GT, bool PAGED>
__device__ __forceinline__ void step_records(const DecodeArgs& a, long long u, const uint8_t* ubase, int g0,
                                             int ns, const uint8_t* (&rp)[4], int (&hf)[4]) {
  constexpr BlockLayout BL = block_layout(KB, VB, GT);
  constexpr int SPB = GT / kStream;  // streams per block
  const uint8_t* const sb = ubase + static_cast<size_t>(g0 / SPB) * BL.bytes;  // (unit-major)
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const int g = min(g0 + gi, g0 + ns - 1);
    hf[gi] = g % SPB;
    if constexpr (PAGED) {
      rp[gi] = a.blocks + record_index(a.page_table, a.page_stride, a.num_pages, a.nb, a.H, u, g / SPB) * BL.bytes;
    } else {
      rp[gi] = sb + (g / SPB - g0 / SPB) * BL.bytes;
    }
  }
}

// The record (and half) of this lane's metadata slot (lanes 16 i .. 16 i +
// 15: stream i), selected with arithmetic rather than branches.
template <int KB, int VB, int GT, bool PAGED>
__device__ __forceinline__ const uint8_t* lane_record(const uint8_t* const (&rp)[4], int g0, int ns, int lane) {
  const int i = lane >> 4;
  if constexpr (PAGED) {
    const uintptr_t r01 = i & 1 ? reinterpret_cast<uintptr_t>(rp[1]) : reinterpret_cast<uintptr_t>(rp[0]);
    const uintptr_t r23 = i & 1 ? reinterpret_cast<uintptr_t>(rp[3]) : reinterpret_cast<uintptr_t>(rp[2]);
    return reinterpret_cast<const uint8_t*>(i & 2 ? r23 : r01);
  } else {
    constexpr BlockLayout BL = block_layout(KB, VB, GT);
    constexpr int SPB = GT / kStream;
    const int g = min(g0 + i, g0 + ns - 1);
    return rp[0] + (g / SPB - g0 / SPB) * BL.bytes;
  }
}
__device__ __forceinline__ int lane_half(int g0, int ns, int spb, int lane) {
  return min(g0 + (lane >> 4), g0 + ns - 1) % spb;
}

// Byte offset, from the record of stream g0, of the record holding stream
// g0 + min(i, ns - 1) and the index of that stream inside its record
// (unit-major records lie BYTES apart).
template <int GT, int BYTES>
__device__ __forceinline__ int stream_record(int g0, int i, int ns, int& half) {
  const int c = min(i, ns - 1);
  if constexpr (GT == kStream) {
    half = 0;
    return c * BYTES;
  } else {
    constexpr int SPB = GT / kStream;
    const int g = g0 + c;
    half = g % SPB;
    return (g / SPB - g0 / SPB) * BYTES;
  }
}

// Key stage of streams [g0, g0 + ns): codes to `dst`, scale and zero to
// `meta`; Stage::kLoads instructions.
template <int KB, int VB, int GT, bool PAGED, bool KEEP>
__device__ __forceinline__ void issue_kstage(const DecodeArgs& a, long long u, const uint8_t* ubase, int g0, int ns,
                                             lds_u8* dst, lds_u8* meta_dst) {
  using S = Stage<KB, VB>;
  constexpr BlockLayout BL = block_layout(KB, VB, GT);
  const int lane = threadIdx.x & 63;
  if constexpr (!PAGED) {
    // unit-major: record offsets from the stream index (uniform), lane
    // offsets in the per-lane operand; no address arithmetic on the vector
    // ALUs beyond the metadata lanes' record
    const __amdgpu_buffer_rsrc_t r = step_rsrc<GT, BL.bytes>(ubase, g0);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      int hf;
      const int rec = stream_record<GT, BL.bytes>(g0, gi, ns, hf) + BL.k_codes + hf * S::kGroup;
#pragma unroll
      for (int j = 0; j < S::kGroup / 1024; ++j)
        dma16_buf<KEEP>(r, lane * 16, rec + j * 1024, dst + gi * S::kGroupPad + j * 1024);
    }
    int hm;
    const int voff = stream_record<GT, BL.bytes>(g0, lane >> 4, ns, hm) + ((lane - 4 * (lane >> 4)) & 15) * 16;
    dma16_buf<KEEP>(r, voff, BL.k_scale, meta_dst);
    dma16_buf<KEEP>(r, voff, BL.k_zero, meta_dst + 4 * D * 2);
    return;
  }
  const uint8_t* rp[4];
  int hf[4];
  step_records<KB, VB, GT, PAGED>(a, u, ubase, g0, ns, rp, hf);
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
#pragma unroll
    for (int j = 0; j < S::kGroup / 1024; ++j)  // a stream's rows: kGroup bytes from row 32 * hf
      dma16<KEEP>(rp[gi] + BL.k_codes + hf[gi] * S::kGroup + j * 1024 + lane * 16, dst + gi * S::kGroupPad + j * 1024);
  }
  // scale and zero of the stream's block: 256 bytes per stream and field, 16
  // lanes per stream.  Stream i's 16-byte chunk j lands in LDS slot
  // (j + 4 i) mod 16 of the stream's 256 bytes: the key wave reads chunk
  // 4 lk + c of four streams at once, which then fall on distinct banks.
  const uint8_t* const meta =
      lane_record<KB, VB, GT, PAGED>(rp, g0, ns, lane) + ((lane - 4 * (lane >> 4)) & 15) * 16;
  dma16<KEEP>(meta + BL.k_scale, meta_dst);
  dma16<KEEP>(meta + BL.k_zero, meta_dst + 4 * D * 2);
}

// Value stage of groups [g0, g0 + ns): Stage::vLoads instructions.
template <int KB, int VB, int GT, bool PAGED, bool KEEP>
__device__ __forceinline__ void issue_vstage(const DecodeArgs& a, long long u, const uint8_t* ubase, int g0, int ns,
                                             lds_u8* dst) {
  using S = Stage<KB, VB>;
  constexpr BlockLayout BL = block_layout(KB, VB, GT);
  const int lane = threadIdx.x & 63;
  if constexpr (!PAGED) {
    const __amdgpu_buffer_rsrc_t r = step_rsrc<GT, BL.bytes>(ubase, g0);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      int hf;
      const int rec = stream_record<GT, BL.bytes>(g0, gi, ns, hf) + BL.v_codes + hf * S::vGroup;
#pragma unroll
      for (int j = 0; j < S::vGroup / 1024; ++j)
        dma16_buf<KEEP>(r, lane * 16, rec + j * 1024, dst + gi * S::vGroup + j * 1024);
    }
    // scale and zero: see below
    const int c = lane & 15;
    int hm;
    const int voff = stream_record<GT, BL.bytes>(g0, lane >> 4, ns, hm) +
                     ((32 * (c >> 2)) / GT * GT + kStream * hm + 8 * (c & 3)) * 2;
    dma16_buf<KEEP>(r, voff, BL.v_scale, dst + S::offVS);
    dma16_buf<KEEP>(r, voff, BL.v_zero, dst + S::offVZ);
    return;
  }
  const uint8_t* rp[4];
  int hf[4];
  step_records<KB, VB, GT, PAGED>(a, u, ubase, g0, ns, rp, hf);
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
#pragma unroll
    for (int j = 0; j < S::vGroup / 1024; ++j)  // the stream's words: vGroup bytes from word row hf * VB
      dma16<KEEP>(rp[gi] + BL.v_codes + hf[gi] * S::vGroup + j * 1024 + lane * 16, dst + gi * S::vGroup + j * 1024);
  }
  // scale and zero of the stream's 32 tokens, stage layout [stream][4 channel
  // groups of 32][32 tokens]; a block stores [D / G][G], so with G = 64 two
  // channel groups of 32 share one stored group.  Lane: stream lane / 16,
  // channel group c / 4 and 8 tokens (c % 4) of c = lane % 16.
  const int c = lane & 15;
  const int off = ((32 * (c >> 2)) / GT * GT + kStream * lane_half(g0, ns, GT / kStream, lane) + 8 * (c & 3)) * 2;
  const uint8_t* const meta = lane_record<KB, VB, GT, PAGED>(rp, g0, ns, lane) + off;
  dma16<KEEP>(meta + BL.v_scale, dst + S::offVS);
  dma16<KEEP>(meta + BL.v_zero, dst + S::offVZ);
}

// ---------------------------------------------------------------------------
// Operand range.  The folded operands q''*S (keys) and p'*S (values) are fp16
// hi + lo pairs, so they must stay below 65504, and the lo half keeps its
// precision only while it stays above the fp16 subnormal range.  Each
// workgroup scales them by powers of two: q'' = q 2^-Ek (one exponent per
// head, from the head's largest |q| and the largest key scale of the records
// the split reads) and p' = p 2^-Ev (one per split, from the largest value
// scale), chosen so that the largest product lies in [2^14, 2^15): Ek and Ev
// are negative for ordinary inputs (the operands are scaled up) and positive
// only for scales and queries near the fp16 limit.  Scaling by a power of
// two is exact; the scores take 2^Ek back in fp32, and the partial's (m, l,
// o) carry 2^-Ev in l and o, which the partial's m + Ev compensates in the
// merge's weights 2^(m - M).

// Largest stored key scale and value scale over the block records of
// streams [gb, ge) of unit u (the same on every lane of the wave).
template <int GT, bool PAGED>
__device__ __forceinline__ void split_scale_max(const DecodeArgs& a, long long u, int gb, int ge, float& sk,
                                                float& sv) {
  constexpr int SPB = GT / kStream;
  const int lane = threadIdx.x & 63;
  const int blk0 = gb / SPB, blk1 = (ge - 1) / SPB;
  uint32_t mk = 0, mv = 0;
  for (int base = blk0; base <= blk1; base += 256) {
    uint32_t e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // four independent loads in flight per lane
      const int blk = base + lane + 64 * i;
      long long r = 0;
      if (blk <= blk1) {
        if constexpr (PAGED) {
          r = record_index(a.page_table, a.page_stride, a.num_pages, a.nb, a.H, u, blk);
        } else {
          r = u * a.nb + blk;
        }
      }
      e[i] = blk <= blk1 ? a.scale_max[r] : 0u;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mk = max(mk, e[i] & 0xffffu);
      mv = max(mv, e[i] >> 16);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mk = max(mk, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mk), off)));
    mv = max(mv, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mv), off)));
  }
  sk = __half2float(__ushort_as_half(static_cast<uint16_t>(mk)));
  sv = __half2float(__ushort_as_half(static_cast<uint16_t>(mv)));
}

// First stream of step `step` of a split over streams [gb, ge) in n_steps
// steps of 4.  Each workgroup walks its steps starting at step `rot`
// (wrapping around): the workgroups of one launch all stream at the same
// rate, and in lock step at equal offsets inside their chunks their loads
// crowd the same memory channels (measured on MI355X: a launch of 1536
// workgroups streaming 12 KiB steps reads 5.1 TB/s in lock step and 6.7 TB/s
// with rotated starts).  The online softmax takes the steps in any order.
__device__ __forceinline__ int step_first(int gb, int step, int n_steps, int rot) {
  int k = step + rot;
  if (k >= n_steps) k -= n_steps;
  return gb + 4 * k;
}

// Wave priority by progress.  Six workgroups share a CU and waves of equal
// priority issue oldest first, so with fixed priorities the workgroups of
// one launch progress at different rates by their dispatch order: measured
// on MI355X with per-workgroup timestamps (c2 decode, 43 steps each), the
// first and third workgroup of each CU finished after 124 us, the second and
// fourth after 180 us, whose value waves shared a SIMD with two key waves;
// the launch lasts as long as its slowest workgroup.  A wave in the first
// half of its steps therefore issues ahead of waves in their second half,
// so workgroups that run ahead yield to those behind; within a half the key
// wave leads, since the value wave waits at every step's barrier for its
// softmax.  (Measured: c2 decode 187 -> 184 us back to back, 172 -> 169 us
// after idle; c1 -2%; rotating priorities or four progress bands balanced
// the workgroups as well but gained no more.)
template <bool KEY>
__device__ __forceinline__ void progress_prio(int step, int n_steps) {
  if (2 * step < n_steps) {
    __builtin_amdgcn_s_setprio(KEY ? 3 : 2);
  } else {
    __builtin_amdgcn_s_setprio(KEY ? 1 : 0);
  }
}

// Smallest E with x * 2^-E < 2^15 (x >= 0 finite), at least -30 (x = 0 and
// tiny x take -30).
__device__ __forceinline__ int range_exp(float x) { return max(-30, __builtin_amdgcn_frexp_expf(x) - 15); }

// ---------------------------------------------------------------------------
// Key wave: scores of each step on the matrix cores, online softmax, and the
// probabilities handed to the value wave.  Writes m and l of the partial.
template <int KB, int VB, bool BF16, int NQ, int GT, bool PAGED, bool KEEP>
__device__ __forceinline__ void key_wave(const DecodeArgs& a, long long u, int b, int h0, int split,
                                         int gb, int ge, int n_steps, int rot, uint8_t* smem, lds_u8* lsm) {
  using S = Stage<KB, VB>;
  using KS = CodeScale<KB>;
  constexpr int KL = KB;  // key words per lane (32 channels)
  const int lane = threadIdx.x & 63;
  const int lc = lane & 15, lk = lane >> 4;
  const int hq = lc >> 2;  // head slot of this lane's B / C columns
  const int jt = lc & 3;
  // With fewer than 3 heads per kv head, head slots hq >= NQ are free: slot
  // NQ + h carries the lo half of head h's q'' * S, so one product per code
  // block takes both halves (half the products); the two columns' sums are
  // added before the softmax.  With 4 heads each column holds hi, then lo.
  constexpr bool kHiLoCols = NQ <= 2;
  // With 4 heads the operands swap roles: A (rows) is the dense operand,
  // row m = 8 s + 2 h + part holding half `part` of head h's q'' * S for
  // stream s of a pair of streams, and B (columns) holds the codes of 16
  // tokens, 8 of each stream of the pair.  One product then takes both
  // halves, and the hi and lo sums of a score land in the same output lane
  // (rows 4 lk .. 4 lk + 3: head 2 (lk & 1) and 2 (lk & 1) + 1, hi then lo),
  // where they are added.  Two dense operands (stream pairs 0-1 and 2-3)
  // serve 8 products per code block: 32 per step instead of 64.  (Not with
  // 4-bit keys and 2-bit values: that variant runs 3 waves per SIMD, and the
  // paired layout's registers spill there inside the step loop.)
  constexpr bool kPairRows = NQ == 4 && !(KB == 4 && VB == 2);
  const int hsrc = kHiLoCols ? hq % NQ : kPairRows ? (lc >> 1) & 3 : hq;  // head whose q this lane takes
  const int part = kHiLoCols ? hq / NQ : kPairRows ? lc & 1 : 0;  // 0: hi, 1: lo, 2 and 3 (NQ = 1): unused

  constexpr BlockLayout BLu = block_layout(KB, VB, GT);
  const uint8_t* const ubase = a.blocks + static_cast<size_t>(u) * a.nb * BLu.bytes;  // (unit-major)
  // the first stage's loads go out before q is read: their latencies overlap
  {
    const int f0 = step_first(gb, 0, n_steps, rot);
    issue_kstage<KB, VB, GT, PAGED, KEEP>(a, u, ubase, f0, min(4, ge - f0), lsm, lsm + S::offKM0);
  }
  // q of head hsrc, channels 32*lk .. 32*lk+31 (unused head slots: zeros)
  float qf[32];
  if (kHiLoCols ? part < 2 : hq < NQ) {
    const uint16_t* qp = a.q + ((long long)b * a.Hq + h0 + hsrc) * D + 32 * lk;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + i);
      const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[i + 2 * e] = to_f32<BF16>(static_cast<uint16_t>(ww[e]));
        qf[i + 2 * e + 1] = to_f32<BF16>(static_cast<uint16_t>(ww[e] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) qf[i] = 0.0f;
  }
  // operand range exponents: Ek for head hq, Ev for the split
  float sk_max, sv_max;
  split_scale_max<GT, PAGED>(a, u, gb, ge, sk_max, sv_max);
  float qabs = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) qabs = fmaxf(qabs, fabsf(qf[i]));
  qabs = swap_max<16>(qabs);
  qabs = swap_max<32>(qabs);  // the 128 channels of head hsrc
  // q'' = q 2^-Ek and q'' S below 2^15 (q'' itself too, when the scales are
  // below 1); p' = p 2^-Ev <= 2^-Ev and p' S below 2^15
  const int ek = range_exp(qabs * fmaxf(sk_max, 1.0f));
  const int ev = range_exp(sv_max);
  // the exponent of head hq, whose scores this lane reads in the softmax
  // (lane 2 hq holds head hq's in the paired-rows layout)
  const int ek_r = kPairRows ? __shfl(ek, 2 * hq) : ek;
  // q'' as fp16 pairs (pair p: channels 2p, 2p+1).  The power-of-two factor
  // keeps q'' exact (a bf16 q is rounded to fp16 once).
  // softmax_scale * log2(e) * 2^Ek multiplies the scores afterwards.  Head
  // slots hq >= NQ carry q'' = 0 and are masked out of the softmax.
  // Pair 4c + a holds channels 8c + a and 8c + a + 4 of the lane's 32 (a =
  // 0..3), the pairing of the codes (see codes8).
  uint32_t q2[16];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      q2[4 * c + a] = pk_rne(__builtin_amdgcn_ldexpf(qf[8 * c + a], -ek), __builtin_amdgcn_ldexpf(qf[8 * c + a + 4], -ek));
  // lo columns (kHiLoCols): B = RN(q'' S - RN(qm S)) with qm = q'' gives the
  // lo half and qm = 0 the hi half, two packed instructions either way
  const uint32_t qmask = ((kHiLoCols || kPairRows) && part == 1) ? 0xffffffffu : 0u;
  // raw product -> score: products are c q S 2^(F-15-Ek)
  const float k_unscale = __builtin_amdgcn_ldexpf(a.qscale, 15 - KS::F + ek_r);
  const float z_unscale = __builtin_amdgcn_ldexpf(a.qscale, ek);  // (the zero-point term of head hsrc)

  const bool diag = (lc & 3) == lk;  // lane holds scores (stream lk)
  float m_run = -INFINITY;           // running max of head hq (base 2)
  float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // sum of p' (four partial sums)

  auto one_step = [&](int step, auto par) __attribute__((always_inline)) {
    const int PAR = parity(step, par);
    progress_prio<true>(step, n_steps);
    const int g0 = step_first(gb, step, n_steps, rot);
    const int ns = min(4, ge - g0);
    // this step's codes and metadata are the only loads of this wave in flight
    wait_vm<0>();
    wave_lds_sync();
    const uint8_t* const meta = smem + S::offKM0 + PAR * S::kMetaBytes;

    // chunk 4 lk + c of stream st sits in slot 4 ((lk + st) mod 4) + c
    auto meta_chunks = [&](int field, int st) {
      return reinterpret_cast<const u32x4*>(meta + field * 4 * D * 2 + st * D * 2 + 64 * ((lk + st) & 3));
    };
    // scale chunks of the lane's dense operand(s) and zero chunks of its
    // zero-point term.  Default layout: stream lc & 3 for both.  Paired
    // rows: scales of stream lc >> 3 of each pair; the zero-point term of
    // head hsrc and stream 2 (lc & 1) + (lc >> 3), so the 16 lanes of a k
    // block cover the 16 (stream, head) terms.
    const int gs0 = kPairRows ? lc >> 3 : lc & 3;
    const u32x4* sBp = meta_chunks(0, gs0);
    const u32x4* sBp1 = meta_chunks(0, gs0 + 2);
    const u32x4* zBp = meta_chunks(1, kPairRows ? 2 * (lc & 1) + (lc >> 3) : lc & 3);
    // code rows: default, tile s holds token 4 s + (lc & 3) of stream lc >> 2
    // (A rows); paired rows, tile 4 P + j holds token 4 (lc & 7) + j of
    // stream 2 P + (lc >> 3) (B columns)
    const uint8_t* krow = kPairRows ? smem + (lc >> 3) * S::kGroupPad + 4 * (lc & 7) * S::kRow + 4 * KL * lk
                                    : smem + (lc >> 2) * S::kGroupPad + (lc & 3) * S::kRow + 4 * KL * lk;
    uint32_t kw[8][KL];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int off = kPairRows ? (s >> 2) * 2 * S::kGroupPad + (s & 3) * S::kRow : 4 * s * S::kRow;
      if constexpr (KL == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(krow + off);
        kw[s][0] = v[0];
        kw[s][1] = v[1];
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(krow + off);
#pragma unroll
        for (int i = 0; i < KL; ++i) kw[s][i] = v[i];
      }
    }
    // the codes are in registers: refill the code buffer (and the other
    // metadata buffer, last read by the previous step) with the next step
    wave_lds_sync();
    if (step + 1 < n_steps) {
      const int g1 = step_first(gb, step + 1, n_steps, rot);
      issue_kstage<KB, VB, GT, PAGED, KEEP>(a, u, ubase, g1, min(4, ge - g1), lsm,
                                            lsm + S::offKM0 + (1 - PAR) * S::kMetaBytes);
    }
    // B = q' * S (hi, lo) for head hq and group g0 + gc, built per block of
    // 32 channels right before its products (the vector work of block c+1
    // overlaps the matrix products of block c); zero-point term
    // sum_d q'_d Z_d of the same (head, group) on the vector ALUs, added to
    // the scores afterwards
    float bcls[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // four partial sums
    f32x4 sc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) sc[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // scale and zero of 8 channels as the pairs (a, a + 4), a = 0..3, of q2
      // and the codes: the record stores them interleaved in that order
      const u32x4 sB = sBp[c], zB = zBp[c];
      const uint32_t sx[4] = {sB[0], sB[1], sB[2], sB[3]};
      const uint32_t zx[4] = {zB[0], zB[1], zB[2], zB[3]};
      u32x4 h4, l4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t qq = q2[4 * c + e];
        uint32_t hi, lo;
        if constexpr (kHiLoCols || kPairRows) {
          hi = residual_pair(qq, sx[e], qq & qmask);  // this lane's half (pair 0 in paired rows)
          lo = 0u;
        } else {
          mul_pair_exact(qq, sx[e], hi, lo);
        }
        h4[e] = hi;
        l4[e] = lo;
        bcls[e] = dot2_acc(qq, zx[e], bcls[e]);
      }
      if constexpr (kPairRows) {
        // the dense operand of streams 2 and 3 (l4)
        const u32x4 sB1 = sBp1[c];
        const uint32_t sx1[4] = {sB1[0], sB1[1], sB1[2], sB1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) l4[e] = residual_pair(q2[4 * c + e], sx1[e], q2[4 * c + e] & qmask);
      }
      half8_t ak[8];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        ak[s] = (KB == 4) ? codes8<4, 0>(kw[s][c & (KL - 1)])
                : (c & 1) ? codes8<2, 1>(kw[s][c >> 1]) : codes8<2, 0>(kw[s][c >> 1]);
      const half8_t bh = as_h8(h4);
      if constexpr (kPairRows) {
        const half8_t bh1 = as_h8(l4);
#pragma unroll
        for (int s = 0; s < 4; ++s) sc[s] = mfma(bh, ak[s], sc[s]);
#pragma unroll
        for (int s = 4; s < 8; ++s) sc[s] = mfma(bh1, ak[s], sc[s]);
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) sc[s] = mfma(ak[s], bh, sc[s]);
        if constexpr (!kHiLoCols) {
          const half8_t bl = as_h8(l4);
#pragma unroll
          for (int s = 0; s < 8; ++s) sc[s] = mfma(ak[s], bl, sc[s]);
        }
      }
    }
    float bias = (bcls[0] + bcls[1]) + (bcls[2] + bcls[3]);
    bias = swap_sum<16>(bias);
    bias = swap_sum<32>(bias) * z_unscale;  // all 128 channels: head hsrc, the zero-point stream

    // ------------------------------------------------------------- softmax
    // The 16 diagonal lanes hold the step's 512 scores (head hq, stream lk,
    // 32 tokens each).  They pass through this step's hand-over buffer (its
    // previous contents were consumed by the value wave two steps ago) so
    // that every lane takes 8 of them: lane (hq, j = lc & 3, lk) owns tokens
    // 8j .. 8j+7 of stream lk, and overwrites them with their probabilities.
    // Rows of 32 scores are padded to kRowP floats: the 16 rows start on
    // distinct banks.
    float* const sl = reinterpret_cast<float*>(smem + S::offP0 + PAR * S::pBytes);
    // (raw products; each reader applies the scale and its stream's
    // zero-point term to its own 8 scores, and with kHiLoCols adds the lo
    // column, which the diagonal lanes of slot hq + NQ write like a head)
    if constexpr (kPairRows) {
      // lanes whose rows (stream lk >> 1 of the pair) and column (stream
      // lc >> 3) agree hold heads 2 (lk & 1) and 2 (lk & 1) + 1 of tokens
      // 4 (lc & 7) .. + 3 over the pair's 4 tiles: hi + lo
      if ((lc >> 3) == (lk >> 1)) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          f32x4 xa, xb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xa[j] = sc[4 * pr + j][0] + sc[4 * pr + j][1];
            xb[j] = sc[4 * pr + j][2] + sc[4 * pr + j][3];
          }
          float* const dst = sl + ((2 * pr + (lc >> 3)) * GQ + 2 * (lk & 1)) * kRowP + 4 * (lc & 7);
          *reinterpret_cast<f32x4*>(dst) = xa;
          *reinterpret_cast<f32x4*>(dst + kRowP) = xb;
        }
      }
      if (lk == 0) sl[S::offBias / 4 + (2 * (lc & 1) + (lc >> 3)) * GQ + hsrc] = bias;
    } else if (diag) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        *reinterpret_cast<f32x4*>(sl + (lk * GQ + hq) * kRowP + 4 * s) = sc[s];
      sl[S::offBias / 4 + lk * GQ + hq] = bias;
    }
    wave_lds_order();  // the reads below take values written by the diagonal lanes
    const int row = (lk * GQ + hq) * kRowP + 8 * jt;
    float x[8];
    {
      f32x4 x0 = *reinterpret_cast<const f32x4*>(sl + row);
      f32x4 x1 = *reinterpret_cast<const f32x4*>(sl + row + 4);
      if constexpr (kHiLoCols) {
        // the lo column's sums of head hq sit in head slot hq + NQ's row
        // (lanes of slots hq >= NQ read a row of their own and are masked)
        const int lrow = (lk * GQ + ((hq + NQ) & (GQ - 1))) * kRowP + 8 * jt;
        x0 += *reinterpret_cast<const f32x4*>(sl + lrow);
        x1 += *reinterpret_cast<const f32x4*>(sl + lrow + 4);
      }
      // streams past the last group hold no tokens; slots hq >= NQ no head.
      // Their raw sums are finite (the stage repeats the last stream's
      // words; unused slots multiply zeros), so a zero-point term of -inf
      // masks all 8 scores.
      const bool valid = lk < ns && hq < NQ;
      const float bz = valid ? sl[S::offBias / 4 + lk * GQ + hq] : -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = fmaf(x0[i], k_unscale, bz);
        x[4 + i] = fmaf(x1[i], k_unscale, bz);
      }
    }
    float mx = max_raw(max_raw(max_raw(x[0], x[1]), max_raw(x[2], x[3])),
                       max_raw(max_raw(x[4], x[5]), max_raw(x[6], x[7])));
    mx = max_raw(mx, partner<1>(mx));
    mx = max_raw(mx, partner<2>(mx));
    mx = swap_max<16>(mx);
    mx = swap_max<32>(mx);  // max over the 4 streams and 32 tokens of head hq
    const float m_new = fmaxf(m_run, mx);
    // rescale factor of the running sums; exactly 1 when the max holds
    const float alpha = !(m_new > m_run) ? 1.0f : (m_run == -INFINITY ? 0.0f : fast_exp2(m_run - m_new));
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < 4; ++e) lsum[e] *= alpha;
    // p' = p 2^-Ev = 2^(x - (m + Ev))
    const float mm = m_run + static_cast<float>(ev);
    f32x4 p0, p1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[i] = fast_exp2(x[i] - mm);
      p1[i] = fast_exp2(x[4 + i] - mm);
    }
    lsum[0] += p0[0] + p0[1];
    lsum[1] += p0[2] + p0[3];
    lsum[2] += p1[0] + p1[1];
    lsum[3] += p1[2] + p1[3];
    *reinterpret_cast<f32x4*>(sl + row) = p0;
    *reinterpret_cast<f32x4*>(sl + row + 4) = p1;
    if (lk == 0 && jt == 0) sl[S::offAlpha / 4 + hq] = alpha;
    wg_barrier();  // step's probabilities ready
  };
  run_steps<!(KB == 4 && VB == 2)>(n_steps, one_step);

  float l = (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
  l = l + partner<1>(l);
  l = l + partner<2>(l);
  l = swap_sum<16>(l);
  l = swap_sum<32>(l);  // the 16 lanes of head hq
  if (lk == 0 && jt == 0 && hq < NQ) {
    // l and the value wave's o carry 2^-Ev; m + Ev restores their weight
    float* P = a.partial + (((long long)b * a.Hq + h0 + hq) * a.n_split + split) * (D + 2);
    P[0] = m_run + static_cast<float>(ev);
    P[1] = l;
  }
}

// ---------------------------------------------------------------------------
// Value wave: p.V of each step on the matrix cores, one step behind the key
// wave.  Writes o of the partial; the last split also runs the window.
template <int KB, int VB, bool BF16, int NQ, int GT, bool PAGED, bool KEEP>
__device__ __forceinline__ void value_wave(const DecodeArgs& a, long long u, int b, int h0, int split,
                                           int gb, int ge, int n_steps, int rot, uint8_t* smem, lds_u8* lsm) {
  using S = Stage<KB, VB>;
  using VS = CodeScale<VB>;
  const int lane = threadIdx.x & 63;
  const int lc = lane & 15, lk = lane >> 4;
  const int hq = lc >> 2;
  const int mcol = lc & 3;  // channel group of this lane's B column
  // With fewer than 3 heads per kv head, head slots hq >= NQ are free: slot
  // NQ + h carries the lo half of head h's p * S, so one product per channel
  // block takes both halves (half the products); the two columns' sums are
  // added once at the end.  With 4 heads each column holds hi, then lo.
  constexpr bool kHiLoCols = NQ <= 2;
  const int hsrc = kHiLoCols ? hq % NQ : hq;  // head whose probabilities this column takes
  const int part = kHiLoCols ? hq / NQ : 0;   // 0: hi, 1: lo, 2 and 3 (NQ = 1): unused
  const uint32_t pmask = (part & 1) ? 0xffffffffu : 0u;  // (kHiLoCols) this column's half, see products
  uint8_t* const vbase = smem + S::offV0;
  lds_u8* const lvbase = lsm + S::offV0;
  constexpr BlockLayout BLu = block_layout(KB, VB, GT);
  const uint8_t* const ubase = a.blocks + static_cast<size_t>(u) * a.nb * BLu.bytes;  // (unit-major)
  {
    const int f0 = step_first(gb, 0, n_steps, rot);
    issue_vstage<KB, VB, GT, PAGED, KEEP>(a, u, ubase, f0, min(4, ge - f0), lvbase);
  }
  constexpr float v_unscale = static_cast<float>(1 << (15 - VS::F));  // product -> output

  float zcls[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // sum of p' * Z (four partial sums)
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto one_step = [&](int step, auto par) __attribute__((always_inline)) {
    const int PAR = parity(step, par);
    progress_prio<false>(step, n_steps);
    const uint8_t* vstage = vbase + PAR * S::vBytes;
    const bool more = step + 1 < n_steps;
    if (more) {
      const int g1 = step_first(gb, step + 1, n_steps, rot);
      issue_vstage<KB, VB, GT, PAGED, KEEP>(a, u, ubase, g1, min(4, ge - g1), lvbase + (1 - PAR) * S::vBytes);
    }
    wg_barrier();  // the key wave has written this step's probabilities
    if (more) {
      wait_vm<S::vLoads>();
    } else {
      wait_vm<0>();
    }
    wave_lds_sync();
    const float* hp = reinterpret_cast<const float*>(smem + S::offP0 + PAR * S::pBytes);
    const float alpha = hp[S::offAlpha / 4 + hsrc];
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) zcls[e] *= alpha;
    }
    // p.V of 32 tokens (one MFMA k block): p0, p1 the probabilities of this
    // lane's 8 tokens, vs / vz their scales and zeros (channel group mcol,
    // token t in half t & 1 of element t / 2), av the codes (entry pairs
    // (a, a + 4), see codes8).  B = p * S as fp16 hi + lo of the binary32
    // product (the probabilities are not exact in fp16, so the product is
    // formed in binary32 and split).  (Handing p over as fp16 hi + lo pairs
    // instead, for packed fp16 products here, takes 48 fewer instructions in
    // this wave and 16 more in the key wave, and measured 3% slower: the key
    // wave sets the pace.)
    auto products = [&](const f32x4& p0, const f32x4& p1, const u32x4& vs, const u32x4& vz, const half8_t (&av)[8]) {
      const float p[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      u32x4 h4, l4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // pair e: tokens e and e + 4
        uint32_t hi, lo;
        const float b0 = (e & 1) ? times_half<1>(p[e], vs[e >> 1]) : times_half<0>(p[e], vs[e >> 1]);
        const float b1 = (e & 1) ? times_half<1>(p[e + 4], vs[2 + (e >> 1)]) : times_half<0>(p[e + 4], vs[2 + (e >> 1)]);
        if constexpr (kHiLoCols) {
          // this lane's half only: RN(b - RN(b) & mask), the hi half with
          // mask 0 and the lo half with mask ~0 (columns of slots past the lo
          // ones take either; their sums are never read)
          hi = pk_rne(b0, b1);
          const uint32_t hm = hi & pmask;
          h4[e] = pk_rne(minus_half<0>(hm, b0), minus_half<1>(hm, b1));
        } else {
          split_pair(b0, b1, hi, lo);
          h4[e] = hi;
          l4[e] = lo;
        }
        zcls[e] = fmaf(p[2 * e], lo_half(vz[e]), zcls[e]);
        zcls[e] = fmaf(p[2 * e + 1], hi_half(vz[e]), zcls[e]);
      }
      if constexpr (kHiLoCols) {
        const half8_t bp = as_h8(h4);
#pragma unroll
        for (int be = 0; be < 8; ++be) o[be] = mfma(av[be], bp, o[be]);
      } else {
        const half8_t bph = as_h8(h4), bpl = as_h8(l4);
#pragma unroll
        for (int be = 0; be < 8; ++be) o[be] = mfma(av[be], bph, o[be]);
#pragma unroll
        for (int be = 0; be < 8; ++be) o[be] = mfma(av[be], bpl, o[be]);
      }
    };
    // All 4 streams, also past the split's last group: the key wave hands
    // over p = 0 there and the stage repeats the last stream's words, so
    // those products add zeros; the unrolled streams form one schedule.
    // Words of channels 4 lc .. 4 lc + 3 and 64 + 4 lc .. 64 + 4 lc + 3: the
    // 16 lanes of a read cover 256 contiguous bytes.
    if constexpr (VB == 2) {
      // A 2-bit word holds 16 tokens (two runs of 8).  Streams go in pairs:
      // lanes of k block lk take word lk & 1 of stream 2 pp + lk / 2, both
      // of its runs (one product block each), so each word read serves 16
      // codes.
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int gsl = 2 * pp + (lk >> 1), w = lk & 1;
        const uint8_t* vrow = vstage + gsl * S::vGroup + (w * D + 4 * lc) * 4;
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(vrow);
        const u32x4 v1 = *reinterpret_cast<const u32x4*>(vrow + 64 * 4);
        const uint32_t vc[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          const int t0 = 16 * w + 8 * run;  // first token of the run in its stream
          const int vmo = ((gsl * 4 + mcol) * G + t0) * 2;
          const u32x4 vs = *reinterpret_cast<const u32x4*>(vstage + S::offVS + vmo);
          const u32x4 vz = *reinterpret_cast<const u32x4*>(vstage + S::offVZ + vmo);
          const float* prow = hp + (gsl * GQ + hsrc) * kRowP + t0;
          const f32x4 p0 = *reinterpret_cast<const f32x4*>(prow);
          const f32x4 p1 = *reinterpret_cast<const f32x4*>(prow + 4);
          half8_t av[8];
#pragma unroll
          for (int be = 0; be < 8; ++be) av[be] = run ? codes8<2, 1>(vc[be]) : codes8<2, 0>(vc[be]);
          products(p0, p1, vs, vz, av);
        }
      }
    } else {
      // a 4-bit word holds one run of 8 tokens: k block lk takes word lk
#pragma unroll
      for (int gs = 0; gs < 4; ++gs) {
        const uint8_t* vrow = vstage + gs * S::vGroup + (lk * D + 4 * lc) * 4;
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(vrow);
        const u32x4 v1 = *reinterpret_cast<const u32x4*>(vrow + 64 * 4);
        const uint32_t vc[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        const int vmo = ((gs * 4 + mcol) * G + 8 * lk) * 2;
        const u32x4 vs = *reinterpret_cast<const u32x4*>(vstage + S::offVS + vmo);
        const u32x4 vz = *reinterpret_cast<const u32x4*>(vstage + S::offVZ + vmo);
        const float* prow = hp + (gs * GQ + hsrc) * kRowP + 8 * lk;
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(prow);
        const f32x4 p1 = *reinterpret_cast<const f32x4*>(prow + 4);
        half8_t av[8];
#pragma unroll
        for (int be = 0; be < 8; ++be) av[be] = codes8<4, 0>(vc[be]);
        products(p0, p1, vs, vz, av);
      }
    }
  };
  run_steps<!(KB == 4 && VB == 2)>(n_steps, one_step);

  float z = (zcls[0] + zcls[1]) + (zcls[2] + zcls[3]);
  z = swap_sum<16>(z);
  z = swap_sum<32>(z);  // sum over the 4 row chunks: head hq, channel group lc & 3
  if constexpr (kHiLoCols) {
    // the lo column of head hq (< NQ) is 4 NQ lanes further in the row of 16
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[i][r] += __shfl_down(o[i][r], 4 * NQ, 16);
  }
  // Row 4 lk + r of product be is channel 16 lk + 4 r + be (be < 4) or
  // 64 + 16 lk + 4 r + be - 4 (be >= 4), of channel group lk / 2 or
  // 2 + lk / 2; the lane whose column holds that group writes it.
  const int mh = (lc & 3) == (lk >> 1) ? 0 : (lc & 3) == 2 + (lk >> 1) ? 1 : -1;
  if (mh >= 0 && hq < NQ) {
    float* P = a.partial + (((long long)b * a.Hq + h0 + hq) * a.n_split + split) * (D + 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = fmaf(mh == 0 ? o[i][r] : o[4 + i][r], v_unscale, z);
      *reinterpret_cast<f32x4*>(P + 2 + 64 * mh + 16 * lk + 4 * r) = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Eight query heads per workgroup (8 or 16 per kv head).  The key products
// put the dense operand in the rows, 8 heads x (hi, lo) = all 16, and the
// codes of 16 tokens of one stream in the columns, so no product is wasted
// and the codes of a record are converted once for all 8 heads (with 4 heads
// per workgroup two workgroups converted them each).  Output lane (lk, lc)
// then holds, for token lc of each (stream, tile of 16 tokens), the hi and
// lo sums of heads 2 lk and 2 lk + 1: its 16 scores, no LDS round trip.  The
// value products keep the codes as rows (16 channels, two channel groups per
// tile) and take as columns 8 heads x the tile's 2 channel groups: half of
// each product's sums are used (a quarter with 4 heads).
template <int KB, int VB, bool BF16, int GT, bool PAGED, bool KEEP>
__device__ __forceinline__ void key_wave8(const DecodeArgs& a, long long u, int b, int h0, int split,
                                          int gb, int ge, int n_steps, int rot, uint8_t* smem, lds_u8* lsm) {
  using S = Stage<KB, VB, 8>;
  using KS = CodeScale<KB>;
  constexpr int KL = KB;  // key words per lane (32 channels)
  const int lane = threadIdx.x & 63;
  const int lc = lane & 15, lk = lane >> 4;
  const int hr = lc >> 1, part = lc & 1;  // A row lc: half `part` of head hr's q'' * S
  constexpr BlockLayout BLu = block_layout(KB, VB, GT);
  const uint8_t* const ubase = a.blocks + static_cast<size_t>(u) * a.nb * BLu.bytes;  // (unit-major)
  {
    const int f0 = step_first(gb, 0, n_steps, rot);
    issue_kstage<KB, VB, GT, PAGED, KEEP>(a, u, ubase, f0, min(4, ge - f0), lsm, lsm + S::offKM0);
  }
  // q of head hr, channels 32 lk .. 32 lk + 31
  float qf[32];
  {
    const uint16_t* qp = a.q + ((long long)b * a.Hq + h0 + hr) * D + 32 * lk;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + i);
      const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[i + 2 * e] = to_f32<BF16>(static_cast<uint16_t>(ww[e]));
        qf[i + 2 * e + 1] = to_f32<BF16>(static_cast<uint16_t>(ww[e] >> 16));
      }
    }
  }
  float sk_max, sv_max;
  split_scale_max<GT, PAGED>(a, u, gb, ge, sk_max, sv_max);
  float qabs = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) qabs = fmaxf(qabs, fabsf(qf[i]));
  qabs = swap_max<16>(qabs);
  qabs = swap_max<32>(qabs);  // the 128 channels of head hr
  const int ek = range_exp(qabs * fmaxf(sk_max, 1.0f));
  const int ev = range_exp(sv_max);
  // exponents of the two heads whose scores this lane holds (lane 2 h has head h's)
  const int ek0 = __shfl(ek, 4 * lk), ek1 = __shfl(ek, 4 * lk + 2);
  uint32_t q2[16];  // pair 4 c + a: channels 8 c + a and 8 c + a + 4 of the lane's 32 (see codes8)
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      q2[4 * c + e] =
          pk_rne(__builtin_amdgcn_ldexpf(qf[8 * c + e], -ek), __builtin_amdgcn_ldexpf(qf[8 * c + e + 4], -ek));
  const uint32_t qmask = part ? 0xffffffffu : 0u;  // hi (RN(q'' S)) or lo (its exact remainder)
  const float k_unscale0 = __builtin_amdgcn_ldexpf(a.qscale, 15 - KS::F + ek0);
  const float k_unscale1 = __builtin_amdgcn_ldexpf(a.qscale, 15 - KS::F + ek1);
  const float z_unscale = __builtin_amdgcn_ldexpf(a.qscale, ek);  // the zero-point terms of head hr

  float m_run[2] = {-INFINITY, -INFINITY};  // running max of heads 2 lk, 2 lk + 1 (base 2)
  float lsum[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};

  for (int step = 0; step < n_steps; ++step) {
    progress_prio<true>(step, n_steps);
    const int g0 = step_first(gb, step, n_steps, rot);
    const int ns = min(4, ge - g0);
    wait_vm<0>();
    wave_lds_sync();
    const uint8_t* const meta = smem + S::offKM0 + (step & 1) * S::kMetaBytes;
    // chunk 4 lk + c of stream st sits in slot 4 ((lk + st) mod 4) + c
    auto meta_chunks = [&](int field, int st) {
      return reinterpret_cast<const u32x4*>(meta + field * 4 * D * 2 + st * D * 2 + 64 * ((lk + st) & 3));
    };
    // codes: B column lc of tile s = 2 g + tt is token 16 tt + lc of stream g
    uint32_t kw[8][KL];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint8_t* row = smem + (s >> 1) * S::kGroupPad + (16 * (s & 1) + lc) * S::kRow + 4 * KL * lk;
      if constexpr (KL == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(row);
        kw[s][0] = v[0];
        kw[s][1] = v[1];
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row);
#pragma unroll
        for (int i = 0; i < KL; ++i) kw[s][i] = v[i];
      }
    }
    wave_lds_sync();
    if (step + 1 < n_steps) {
      const int g1 = step_first(gb, step + 1, n_steps, rot);
      issue_kstage<KB, VB, GT, PAGED, KEEP>(a, u, ubase, g1, min(4, ge - g1), lsm,
                                            lsm + S::offKM0 + ((step + 1) & 1) * S::kMetaBytes);
    }
    // A (per stream and block of 32 channels) = this lane's half of q'' * S;
    // the zero-point terms sum_d q'_d Z_d of head hr and streams 2 part,
    // 2 part + 1 on the vector ALUs
    float bcls[2] = {0.0f, 0.0f};
    f32x4 sc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) sc[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // the codes of a tile are converted right before its products (few
      // registers live)
      auto codes = [&](int s) {
        return (KB == 4) ? codes8<4, 0>(kw[s][c & (KL - 1)])
               : (c & 1) ? codes8<2, 1>(kw[s][c >> 1]) : codes8<2, 0>(kw[s][c >> 1]);
      };
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 sB = meta_chunks(0, g)[c];
        u32x4 h4;
#pragma unroll
        for (int e = 0; e < 4; ++e) h4[e] = residual_pair(q2[4 * c + e], sB[e], q2[4 * c + e] & qmask);
        const half8_t ah = as_h8(h4);
        sc[2 * g] = mfma(ah, codes(2 * g), sc[2 * g]);
        sc[2 * g + 1] = mfma(ah, codes(2 * g + 1), sc[2 * g + 1]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 zB = meta_chunks(1, 2 * part + j)[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) bcls[j] = dot2_acc(q2[4 * c + e], zB[e], bcls[j]);
      }
    }
    float* const sl = reinterpret_cast<float*>(smem + S::offP0 + (step & 1) * S::pBytes);
    // zero-point terms over all 128 channels, exchanged through LDS as [stream][head]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float bz = swap_sum<16>(bcls[j]);
      bz = swap_sum<32>(bz) * z_unscale;
      if (lk == 0) sl[S::offBias / 4 + (2 * part + j) * 8 + hr] = bz;
    }
    wave_lds_order();
    // scores of heads 2 lk (rows 4 lk, 4 lk + 1: hi, lo) and 2 lk + 1 (rows
    // 4 lk + 2, 4 lk + 3) at token 16 (s & 1) + lc of stream s >> 1.
    // Streams past the last group hold no tokens: a zero-point term of -inf
    // masks their scores (their raw sums are finite).
    float x0[8], x1[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 bzw = *reinterpret_cast<const u32x2*>(sl + S::offBias / 4 + g * 8 + 2 * lk);
      const bool valid = g < ns;
      const float bz0 = valid ? __uint_as_float(bzw[0]) : -INFINITY;
      const float bz1 = valid ? __uint_as_float(bzw[1]) : -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 v = sc[2 * g + tt];
        x0[2 * g + tt] = fmaf(v[0] + v[1], k_unscale0, bz0);
        x1[2 * g + tt] = fmaf(v[2] + v[3], k_unscale1, bz1);
      }
    }
    float mx0 = max_raw(max_raw(max_raw(x0[0], x0[1]), max_raw(x0[2], x0[3])),
                        max_raw(max_raw(x0[4], x0[5]), max_raw(x0[6], x0[7])));
    float mx1 = max_raw(max_raw(max_raw(x1[0], x1[1]), max_raw(x1[2], x1[3])),
                        max_raw(max_raw(x1[4], x1[5]), max_raw(x1[6], x1[7])));
    mx0 = row_max16(mx0);  // the 16 lanes of group lk hold all 128 tokens of head 2 lk
    mx1 = row_max16(mx1);
    float alpha[2];
    const float mxs[2] = {mx0, mx1};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float m_new = fmaxf(m_run[i], mxs[i]);
      alpha[i] = !(m_new > m_run[i]) ? 1.0f : (m_run[i] == -INFINITY ? 0.0f : fast_exp2(m_run[i] - m_new));
      m_run[i] = m_new;
      lsum[i][0] *= alpha[i];
      lsum[i][1] *= alpha[i];
    }
    const float mm0 = m_run[0] + static_cast<float>(ev), mm1 = m_run[1] + static_cast<float>(ev);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float p0 = fast_exp2(x0[s] - mm0), p1 = fast_exp2(x1[s] - mm1);
      lsum[0][s & 1] += p0;
      lsum[1][s & 1] += p1;
      float* const pr = sl + ((s >> 1) * 8 + 2 * lk) * kRowP + 16 * (s & 1) + lc;
      pr[0] = p0;
      pr[kRowP] = p1;
    }
    if (lc == 0) {
      sl[S::offAlpha / 4 + 2 * lk] = alpha[0];
      sl[S::offAlpha / 4 + 2 * lk + 1] = alpha[1];
    }
    wg_barrier();  // step's probabilities ready
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float l = row_sum16(lsum[i][0] + lsum[i][1]);
    if (lc == 0) {
      // l and the value wave's o carry 2^-Ev; m + Ev restores their weight
      float* P = a.partial + (((long long)b * a.Hq + h0 + 2 * lk + i) * a.n_split + split) * (D + 2);
      P[0] = m_run[i] + static_cast<float>(ev);
      P[1] = l;
    }
  }
}

template <int KB, int VB, bool BF16, int GT, bool PAGED, bool KEEP>
__device__ __forceinline__ void value_wave8(const DecodeArgs& a, long long u, int b, int h0, int split,
                                            int gb, int ge, int n_steps, int rot, uint8_t* smem, lds_u8* lsm) {
  using S = Stage<KB, VB, 8>;
  using VS = CodeScale<VB>;
  const int lane = threadIdx.x & 63;
  const int lc = lane & 15, lk = lane >> 4;
  // B column lc: head hsrc, channel group msel of tiles 0-3 (channels 0-63)
  // and 2 + msel of tiles 4-7
  const int hsrc = lc >> 1, msel = lc & 1;
  uint8_t* const vbase = smem + S::offV0;
  lds_u8* const lvbase = lsm + S::offV0;
  constexpr BlockLayout BLu = block_layout(KB, VB, GT);
  const uint8_t* const ubase = a.blocks + static_cast<size_t>(u) * a.nb * BLu.bytes;  // (unit-major)
  {
    const int f0 = step_first(gb, 0, n_steps, rot);
    issue_vstage<KB, VB, GT, PAGED, KEEP>(a, u, ubase, f0, min(4, ge - f0), lvbase);
  }
  constexpr float v_unscale = static_cast<float>(1 << (15 - VS::F));  // product -> output

  float za[4] = {0.0f, 0.0f, 0.0f, 0.0f}, zb[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // sums of p' * Z
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int step = 0; step < n_steps; ++step) {
    progress_prio<false>(step, n_steps);
    const uint8_t* vstage = vbase + (step & 1) * S::vBytes;
    const bool more = step + 1 < n_steps;
    if (more) {
      const int g1 = step_first(gb, step + 1, n_steps, rot);
      issue_vstage<KB, VB, GT, PAGED, KEEP>(a, u, ubase, g1, min(4, ge - g1),
                                            lvbase + ((step + 1) & 1) * S::vBytes);
    }
    wg_barrier();  // the key wave has written this step's probabilities
    if (more) {
      wait_vm<S::vLoads>();
    } else {
      wait_vm<0>();
    }
    wave_lds_sync();
    const float* hp = reinterpret_cast<const float*>(smem + S::offP0 + (step & 1) * S::pBytes);
    const float alpha = hp[S::offAlpha / 4 + hsrc];
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        za[e] *= alpha;
        zb[e] *= alpha;
      }
    }
    // p.V of one k block of 32 tokens: p0, p1 this lane's 8 tokens of head
    // hsrc; scale and zero of channel group msel (va*) and 2 + msel (vb*);
    // av the codes (entry pairs (a, a + 4), see codes8)
    auto products = [&](const f32x4& p0, const f32x4& p1, const u32x4& vsa, const u32x4& vza, const u32x4& vsb,
                        const u32x4& vzb, const uint32_t (&vc)[8], int run) {
      const float p[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      u32x4 ha, la, hb, lb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // pair e: tokens e and e + 4
        uint32_t hi, lo;
        float b0 = (e & 1) ? times_half<1>(p[e], vsa[e >> 1]) : times_half<0>(p[e], vsa[e >> 1]);
        float b1 = (e & 1) ? times_half<1>(p[e + 4], vsa[2 + (e >> 1)]) : times_half<0>(p[e + 4], vsa[2 + (e >> 1)]);
        split_pair(b0, b1, hi, lo);
        ha[e] = hi;
        la[e] = lo;
        b0 = (e & 1) ? times_half<1>(p[e], vsb[e >> 1]) : times_half<0>(p[e], vsb[e >> 1]);
        b1 = (e & 1) ? times_half<1>(p[e + 4], vsb[2 + (e >> 1)]) : times_half<0>(p[e + 4], vsb[2 + (e >> 1)]);
        split_pair(b0, b1, hi, lo);
        hb[e] = hi;
        lb[e] = lo;
        za[e] = fmaf(p[2 * e], lo_half(vza[e]), za[e]);
        za[e] = fmaf(p[2 * e + 1], hi_half(vza[e]), za[e]);
        zb[e] = fmaf(p[2 * e], lo_half(vzb[e]), zb[e]);
        zb[e] = fmaf(p[2 * e + 1], hi_half(vzb[e]), zb[e]);
      }
      const half8_t bha = as_h8(ha), bla = as_h8(la), bhb = as_h8(hb), blb = as_h8(lb);
      // each tile's codes converted right before its two products
#pragma unroll
      for (int be = 0; be < 8; ++be) {
        const half8_t av = (VB == 4) ? codes8<4, 0>(vc[be]) : run ? codes8<2, 1>(vc[be]) : codes8<2, 0>(vc[be]);
        o[be] = mfma(av, be < 4 ? bha : bhb, o[be]);
        o[be] = mfma(av, be < 4 ? bla : blb, o[be]);
      }
    };
    // All 4 streams, also past the split's last group (p = 0 there, see value_wave).
    if constexpr (VB == 2) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int gsl = 2 * pp + (lk >> 1), w = lk & 1;
        const uint8_t* vrow = vstage + gsl * S::vGroup + (w * D + 4 * lc) * 4;
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(vrow);
        const u32x4 v1 = *reinterpret_cast<const u32x4*>(vrow + 64 * 4);
        const uint32_t vc[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          const int t0 = 16 * w + 8 * run;  // first token of the run in its stream
          const int vma = ((gsl * 4 + msel) * G + t0) * 2, vmb = ((gsl * 4 + 2 + msel) * G + t0) * 2;
          const u32x4 vsa = *reinterpret_cast<const u32x4*>(vstage + S::offVS + vma);
          const u32x4 vza = *reinterpret_cast<const u32x4*>(vstage + S::offVZ + vma);
          const u32x4 vsb = *reinterpret_cast<const u32x4*>(vstage + S::offVS + vmb);
          const u32x4 vzb = *reinterpret_cast<const u32x4*>(vstage + S::offVZ + vmb);
          const float* prow = hp + (gsl * 8 + hsrc) * kRowP + t0;
          const f32x4 p0 = *reinterpret_cast<const f32x4*>(prow);
          const f32x4 p1 = *reinterpret_cast<const f32x4*>(prow + 4);
          products(p0, p1, vsa, vza, vsb, vzb, vc, run);
        }
      }
    } else {
#pragma unroll
      for (int gs = 0; gs < 4; ++gs) {
        const uint8_t* vrow = vstage + gs * S::vGroup + (lk * D + 4 * lc) * 4;
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(vrow);
        const u32x4 v1 = *reinterpret_cast<const u32x4*>(vrow + 64 * 4);
        const uint32_t vc[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        const int vma = ((gs * 4 + msel) * G + 8 * lk) * 2, vmb = ((gs * 4 + 2 + msel) * G + 8 * lk) * 2;
        const u32x4 vsa = *reinterpret_cast<const u32x4*>(vstage + S::offVS + vma);
        const u32x4 vza = *reinterpret_cast<const u32x4*>(vstage + S::offVZ + vma);
        const u32x4 vsb = *reinterpret_cast<const u32x4*>(vstage + S::offVS + vmb);
        const u32x4 vzb = *reinterpret_cast<const u32x4*>(vstage + S::offVZ + vmb);
        const float* prow = hp + (gs * 8 + hsrc) * kRowP + 8 * lk;
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(prow);
        const f32x4 p1 = *reinterpret_cast<const f32x4*>(prow + 4);
        products(p0, p1, vsa, vza, vsb, vzb, vc, 0);
      }
    }
  }

  float zsa = (za[0] + za[1]) + (za[2] + za[3]);
  float zsb = (zb[0] + zb[1]) + (zb[2] + zb[3]);
  zsa = swap_sum<32>(swap_sum<16>(zsa));  // over the 4 row chunks: head hsrc, channel group msel
  zsb = swap_sum<32>(swap_sum<16>(zsb));  // channel group 2 + msel
  // Row 4 lk + r of product be is channel 16 lk + 4 r + be (be < 4, group
  // lk / 2) or 64 + 16 lk + 4 r + be - 4 (group 2 + lk / 2): the lanes whose
  // column takes group lk / 2 and 2 + lk / 2 write both halves.
  if (msel == (lk >> 1)) {
    float* P = a.partial + (((long long)b * a.Hq + h0 + hsrc) * a.n_split + split) * (D + 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 x, y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = fmaf(o[i][r], v_unscale, zsa);
        y[i] = fmaf(o[4 + i][r], v_unscale, zsb);
      }
      *reinterpret_cast<f32x4*>(P + 2 + 16 * lk + 4 * r) = x;
      *reinterpret_cast<f32x4*>(P + 2 + 64 + 16 * lk + 4 * r) = y;
    }
  }
}

// Workgroup w of the launch (a 1-D grid) -> pair index P = split + nx * row
// over the (split, unit row) pairs, and head group hg.  With one head group
// P = w.  With hg > 1 head groups (16 query heads per kv head: 8 heads per
// workgroup) the workgroups of one pair read the same records; w takes
// them 8 apart, so they fall on the same XCD (workgroups are dealt to the 8
// XCDs in turn) at about the same time and the second one reads the records
// from that XCD's L2:
//   w = (P / 8) * 8 hg + 8 g + P % 8   (g = 0 .. hg - 1).
__device__ __forceinline__ unsigned pair_of(unsigned w, int hg, int& g) {
  if (hg == 1) {
    g = 0;
    return w;
  }
  g = static_cast<int>((w >> 3) % static_cast<unsigned>(hg));
  return (w / (8u * hg)) * 8u + (w & 7u);
}

template <int KB, int VB, bool BF16, int NQ, int GT, bool PAGED, bool KEEP>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(3))) void decode_mfma(DecodeArgs a) {
  constexpr int NH = NQ == 8 ? 8 : GQ;  // head slots of the stage layout
  using S = Stage<KB, VB, NH>;
  __shared__ __align__(16) uint8_t smem[S::bytes];
  lds_u8* const lsm = (lds_u8*)smem;  // (C-style: an address-space conversion)
  const int wave = threadIdx.x >> 6;  // 0: key wave, 1: value wave
  const int nx = a.n_split_packed > 0 ? a.n_split_packed : 1;
  int hgi;
  const unsigned P = pair_of(blockIdx.x, a.hg, hgi);
  if (P >= static_cast<unsigned>(nx) * static_cast<unsigned>(a.B * a.H)) return;  // (grid rounding)
  const int split = static_cast<int>(P % static_cast<unsigned>(nx));
  const int row = static_cast<int>(P / static_cast<unsigned>(nx));
  const int kvh = row % a.H;
  // this unit's sequence and lengths: the launch's, or its own in a ragged launch
  int b = row / a.H, nq = a.n_quant, nr = a.n_resid;
  if (a.ragged) {
    nq = a.seq_len[b][0];
    nr = a.seq_len[b][1];
    b += a.seq0;
  }
  const long long u = (long long)b * a.H + kvh;
  const int h0 = kvh * a.gq + hgi * NQ;  // first query head of this workgroup

  if (a.n_split_packed > 0) {
    const int nqg = nq / kStream;  // packed streams of 32 tokens
    const int gb = split * a.groups_per_split;
    const int ge = min(nqg, gb + a.groups_per_split);
    if (gb >= nqg) {
      // (ragged) this sequence ends before this split: an empty partial
      // (m = -inf, l = 0, o = 0)
      for (int i = threadIdx.x; i < NQ * (D + 2); i += 128) {
        float* Pp = a.partial + (((long long)b * a.Hq + h0 + i / (D + 2)) * a.n_split + split) * (D + 2);
        Pp[i % (D + 2)] = i % (D + 2) == 0 ? -INFINITY : 0.0f;
      }
    } else {
      const int n_steps = (ge - gb + 3) / 4;  // >= 1: every split holds a group
      // the first step of this workgroup's walk (see step_first); the head
      // groups of one pair take the same walk
      const int rot = static_cast<int>(P % static_cast<unsigned>(n_steps));
      // Both waves run the same number of steps and meet at one barrier per step.
      if constexpr (NQ == 8) {
        if (wave == 0) {
          key_wave8<KB, VB, BF16, GT, PAGED, KEEP>(a, u, b, h0, split, gb, ge, n_steps, rot, smem, lsm);
        } else {
          value_wave8<KB, VB, BF16, GT, PAGED, KEEP>(a, u, b, h0, split, gb, ge, n_steps, rot, smem, lsm);
        }
      } else {
        if (wave == 0) {
          key_wave<KB, VB, BF16, NQ, GT, PAGED, KEEP>(a, u, b, h0, split, gb, ge, n_steps, rot, smem, lsm);
        } else {
          value_wave<KB, VB, BF16, NQ, GT, PAGED, KEEP>(a, u, b, h0, split, gb, ge, n_steps, rot, smem, lsm);
        }
      }
    }
  }
  // The window is one more partial (slot n_split_packed), run by the value
  // wave of the last packed split (of the only workgroup when nothing is
  // packed yet); empty for a sequence without window tokens in a ragged
  // launch.  That wave's stage loads have completed, so its value stages
  // serve as scratch.
  if (wave == 1 && a.n_split > a.n_split_packed && split == nx - 1) {
    wave_lds_sync();
    window_wave<BF16, NQ>(a, u, b, h0, a.n_split_packed, nr, hgi == 0,
                          reinterpret_cast<float (*)[D]>(smem + S::offV0),
                          reinterpret_cast<float (*)[G]>(smem + S::offV0 + NH * D * 4));
  }
}

template <int KB, int VB, bool BF16, int NQ, int GT, bool PAGED, bool KEEP>
hipError_t launch_k(const DecodeArgs& a, hipStream_t stream) {
  // one workgroup per packed split (per head group), one split when nothing
  // is packed; the last one also runs the window.  A ragged launch covers
  // a.B sequences from a.seq0.
  const long long pairs = (long long)(a.n_split_packed > 0 ? a.n_split_packed : 1) * a.B * a.H;
  const long long grid = a.hg == 1 ? pairs : (pairs + 7) / 8 * 8 * a.hg;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_mfma<KB, VB, BF16, NQ, GT, PAGED, KEEP>), dim3(static_cast<unsigned>(grid)), dim3(128), 0,
                     stream, a);
  return hipGetLastError();
}

template <int KB, int VB, bool BF16, int NQ, int GT, bool PAGED>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  // head groups (16 query heads per kv head: two workgroups of 8) keep the
  // records in L2
  if constexpr (NQ == 8) {
    if (a.hg > 1) return launch_k<KB, VB, BF16, NQ, GT, PAGED, true>(a, stream);
  }
  return launch_k<KB, VB, BF16, NQ, GT, PAGED, false>(a, stream);
}

template <int KB, int VB, bool BF16, int NQ>
hipError_t launch_gp(const DecodeArgs& a, hipStream_t stream) {
  if (a.G == 64)
    return a.page_table ? launch_t<KB, VB, BF16, NQ, 64, true>(a, stream) : launch_t<KB, VB, BF16, NQ, 64, false>(a, stream);
  return a.page_table ? launch_t<KB, VB, BF16, NQ, 32, true>(a, stream) : launch_t<KB, VB, BF16, NQ, 32, false>(a, stream);
}

template <int KB, int VB, bool BF16>
hipError_t launch_nq(const DecodeArgs& a, hipStream_t stream) {
  // 16 query heads per kv head: 2 head groups of 8 (a.hg)
  if (a.hg != (a.gq > 8 ? a.gq / 8 : 1)) return hipErrorInvalidValue;
  switch (a.gq) {
    case 1: return launch_gp<KB, VB, BF16, 1>(a, stream);
    case 2: return launch_gp<KB, VB, BF16, 2>(a, stream);
    case 4: return launch_gp<KB, VB, BF16, 4>(a, stream);
    case 8:
    case 16: return launch_gp<KB, VB, BF16, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int k_bits, int v_bits, int kv_dtype,
                              hipStream_t stream) {
  const bool bf = kv_dtype == 1;
#define KIVI_MFMA_CASE(KB, VB) \
  if (k_bits == KB && v_bits == VB) return bf ? launch_nq<KB, VB, true>(a, stream) : launch_nq<KB, VB, false>(a, stream);
  KIVI_MFMA_CASE(2, 2)
  KIVI_MFMA_CASE(2, 4)
  KIVI_MFMA_CASE(4, 2)
  KIVI_MFMA_CASE(4, 4)
#undef KIVI_MFMA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kivi
