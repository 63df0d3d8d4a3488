// kivi_decode.hip - split-K decode attention over the packed cache plus the
// residual window, and the cross-split merge.
//
// Method: decode attention must read the whole cache for every new token,
// so it is bound by memory traffic, and the dequantization has to happen
// inside the attention kernel for the smaller cache to pay off (page
// "KV-Cache Quantization: I Ran the Experiments", "Component 1" and "Where it
// still breaks" item 3; page "KIVI: Asymmetric 2-Bit KV Cache Quantization
// Guide", "Production Serving and vLLM Deployment Trade-offs").  Dequantized
// value = code * scale + zero ("Step 2" of the same guide, floating zero).
//
// Work split: grid (n_split, B * H).  A workgroup owns one (batch, kv head)
// unit and a contiguous range of work items: packed blocks of 32 tokens
// first, then 32-token chunks of the residual window.  It serves all gq query
// heads of that kv head, keeps an online softmax in base 2 (q is pre-scaled
// by softmax_scale * log2 e) and writes (m, l, o[D]) per query head and
// split.  The merge kernel combines the splits exactly:
//   M = max m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int G = kGroup;
constexpr int D = kHeadDim;

template <bool BF16>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  } else {
    return __half2float(__ushort_as_half(h));
  }
}

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

template <int BITS>
__device__ __forceinline__ uint32_t code_at(uint32_t word, int i) {
  return (word >> (BITS * (i >> 1) + 16 * (i & 1))) & ((1u << BITS) - 1u);
}

// ---------------------------------------------------------------------------
// Reference-structured VALU kernel: every element is dequantized in fp32 and
// both products run on the vector ALUs.  Work items are 32-token streams: a
// block of GT = 32 tokens, or half of a block of GT = 64 (whose key scale and
// zero both halves share; its key rows, value word rows and value scale/zero
// rows of the half start at row 32 * half).
template <int KB, int VB, bool BF16, int GQ, int GT>
__global__ __launch_bounds__(256) void decode_split_valu(DecodeArgs a) {
  constexpr int PK = 32 / KB, KW = D / PK;
  constexpr int PV = 32 / VB;
  constexpr BlockLayout BL = block_layout(KB, VB, GT);
  constexpr int SPB = GT / kStream;  // streams per block

  __shared__ float qs[GQ][D];
  __shared__ float kS[D], kZ[D];
  __shared__ float vS[D], vZ[D];          // [channel group of GT][row of the block]
  __shared__ float sc[GQ][G];             // scores, then probabilities
  __shared__ float st_m[GQ], st_l[GQ], st_a[GQ];
  __shared__ float ored[GQ][D];

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int h = static_cast<int>(blockIdx.y % a.H);
  // this unit's sequence and lengths: the launch's, or its own in a ragged
  // launch (a split past the sequence's end leaves an empty partial)
  int b = static_cast<int>(blockIdx.y / a.H), nq = a.n_quant, nr = a.n_resid;
  if (a.ragged) {
    nq = a.seq_len[b][0];
    nr = a.seq_len[b][1];
    b += a.seq0;
  }
  const long long u = (long long)b * a.H + h;

  for (int i = tid; i < GQ * D; i += 256) {
    const int j = i / D, d = i % D;
    qs[j][d] = to_f32<BF16>(a.q[((long long)b * a.Hq + h * GQ + j) * D + d]) * a.qscale;
  }
  if (tid < GQ) {
    st_m[tid] = -INFINITY;
    st_l[tid] = 0.0f;
  }
  float o[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) o[j] = 0.0f;

  const int nqb = nq / kStream;  // packed streams
  const int n_items = nqb + (nr + G - 1) / G;
  const int i0 = split * a.items_per_split;
  const int i1 = min(n_items, i0 + a.items_per_split);
  __syncthreads();

  for (int it = i0; it < i1; ++it) {
    const bool packed = it < nqb;
    const int rc = it - nqb;  // window chunk index when !packed
    const int ntok = packed ? G : min(G, nr - rc * G);
    const int r0 = packed ? (it % SPB) * kStream : 0;  // first row of the stream in its block
    const uint8_t* const rec =
        a.blocks + record_index(a.page_table, a.page_stride, a.num_pages, a.nb, a.H, u, packed ? it / SPB : 0) * BL.bytes;
    if (packed) {
      // key meta [d]; value meta [m][row], (D / GT) * GT = D entries
      if (tid < D) {
        kS[tid] = h2f(reinterpret_cast<const uint16_t*>(rec + BL.k_scale)[tid]);
        vS[tid] = h2f(reinterpret_cast<const uint16_t*>(rec + BL.v_scale)[tid]);
      } else {
        kZ[tid - D] = h2f(reinterpret_cast<const uint16_t*>(rec + BL.k_zero)[tid - D]);
        vZ[tid - D] = h2f(reinterpret_cast<const uint16_t*>(rec + BL.v_zero)[tid - D]);
      }
    }
    __syncthreads();

    // ---- scores: token t = tid / 8, channels 16*sl .. 16*sl+15
    {
      const int t = tid >> 3, sl = tid & 7;
      float acc[GQ];
#pragma unroll
      for (int j = 0; j < GQ; ++j) acc[j] = 0.0f;
      if (t < ntok) {
        if (packed) {
          const uint32_t* kw = reinterpret_cast<const uint32_t*>(rec + BL.k_codes) + (r0 + t) * KW;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int d = sl * 16 + i;
            const uint32_t c = code_at<KB>(kw[d / PK], d % PK);
            const float kh = fmaf(static_cast<float>(c), kS[d], kZ[d]);
#pragma unroll
            for (int j = 0; j < GQ; ++j) acc[j] = fmaf(qs[j][d], kh, acc[j]);
          }
        } else {
          const uint16_t* kr = a.k_resid + (u * a.R + rc * G + t) * D + sl * 16;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float kh = to_f32<BF16>(kr[i]);
#pragma unroll
            for (int j = 0; j < GQ; ++j) acc[j] = fmaf(qs[j][sl * 16 + i], kh, acc[j]);
          }
        }
      }
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {
#pragma unroll
        for (int j = 0; j < GQ; ++j) acc[j] += __shfl_xor(acc[j], off);
      }
      if (sl == 0) {
#pragma unroll
        for (int j = 0; j < GQ; ++j) sc[j][t] = (t < ntok) ? acc[j] : -INFINITY;
      }
    }
    __syncthreads();

    // ---- online softmax update, one wave per head
    {
      const int wave = tid >> 6, lane = tid & 63;
      for (int j = wave; j < GQ; j += 4) {
        const float s = lane < G ? sc[j][lane] : -INFINITY;
        float mx = s;
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        const float m_old = st_m[j];
        const float m_new = fmaxf(m_old, mx);
        const float p = (s == -INFINITY) ? 0.0f : exp2f(s - m_new);
        float ps = p;
        for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
        if (lane < G) sc[j][lane] = p;
        if (lane == 0) {
          const float alpha = (m_old == -INFINITY) ? 0.0f : exp2f(m_old - m_new);
          st_l[j] = st_l[j] * alpha + ps;
          st_m[j] = m_new;
          st_a[j] = alpha;
        }
      }
    }
    __syncthreads();

    // ---- values: channel d = tid % 128, rows 16*half .. 16*half+15
    {
      const int d = tid & (D - 1), half = tid >> 7, m = d / GT;
#pragma unroll
      for (int j = 0; j < GQ; ++j) o[j] *= st_a[j];
      if (packed) {
        const uint32_t* vw = reinterpret_cast<const uint32_t*>(rec + BL.v_codes) + d;  // word w at vw[w * D]
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = half * 16 + i, br = r0 + row;  // row of the stream, of the block
          const uint32_t c = code_at<VB>(vw[(br / PV) * D], br % PV);
          const float vh = fmaf(static_cast<float>(c), vS[m * GT + br], vZ[m * GT + br]);
#pragma unroll
          for (int j = 0; j < GQ; ++j) o[j] = fmaf(sc[j][row], vh, o[j]);
        }
      } else {
        for (int i = 0; i < 16; ++i) {
          const int row = half * 16 + i;
          if (row < ntok) {
            const float vh = to_f32<BF16>(a.v_resid[(u * a.R + rc * G + row) * D + d]);
#pragma unroll
            for (int j = 0; j < GQ; ++j) o[j] = fmaf(sc[j][row], vh, o[j]);
          }
        }
      }
    }
    __syncthreads();
  }

  if (tid >= D) {
#pragma unroll
    for (int j = 0; j < GQ; ++j) ored[j][tid - D] = o[j];
  }
  __syncthreads();
  if (tid < D) {
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
      float* P = a.partial + (((long long)b * a.Hq + h * GQ + j) * a.n_split + split) * (D + 2);
      P[2 + tid] = o[j] + ored[j][tid];
      if (tid == 0) {
        P[0] = st_m[j];
        P[1] = st_l[j];
      }
    }
  }
}

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

template <int KB, int VB, bool BF16, int GQ>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_split, a.B * a.H);
  if (a.G == 64) {
    hipLaunchKernelGGL((decode_split_valu<KB, VB, BF16, GQ, 64>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_split_valu<KB, VB, BF16, GQ, 32>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <int KB, int VB, bool BF16>
hipError_t launch_split_gq(const DecodeArgs& a, hipStream_t stream) {
  switch (a.gq) {
    case 1: return launch_split<KB, VB, BF16, 1>(a, stream);
    case 2: return launch_split<KB, VB, BF16, 2>(a, stream);
    case 4: return launch_split<KB, VB, BF16, 4>(a, stream);
    case 8: return launch_split<KB, VB, BF16, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int k_bits, int v_bits, int kv_dtype,
                         int out_dtype, bool use_mfma, hipStream_t stream,
                         hipEvent_t split_begin, hipEvent_t split_end) {
  const bool bf = kv_dtype == 1;
  hipError_t e = hipErrorInvalidValue;
  if (split_begin) {
    e = hipEventRecord(split_begin, stream);
    if (e != hipSuccess) return e;
    e = hipErrorInvalidValue;
  }
  if (use_mfma) {
    e = launch_decode_mfma(a, k_bits, v_bits, kv_dtype, stream);
  } else {
#define KIVI_SPLIT_CASE(KB, VB)                                                   \
  if (k_bits == KB && v_bits == VB)                                               \
    e = bf ? launch_split_gq<KB, VB, true>(a, stream) : launch_split_gq<KB, VB, false>(a, stream);
  KIVI_SPLIT_CASE(2, 2)
  KIVI_SPLIT_CASE(2, 4)
  KIVI_SPLIT_CASE(4, 2)
  KIVI_SPLIT_CASE(4, 4)
#undef KIVI_SPLIT_CASE
  }
  if (e != hipSuccess) return e;
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
