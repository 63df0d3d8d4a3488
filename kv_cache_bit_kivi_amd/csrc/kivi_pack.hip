// kivi_pack.hip - quantize and bit-pack blocks of G = 32 or 64 tokens (keys per
// channel, values per token) and copy tokens into the residual window.
//
// Method: page "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide", "The
// Three Structural Innovations of KIVI" (items 1-3) and "Step 1" (min/max
// scale, half-to-even rounding, clamp); page "KV cache quantization with KIVI
// INT2 setup guide", "KIVI: Per-Channel Key, Per-Token Value Quantization
// Explained" (G = 32, R = 128).  The quantizer itself is in kivi_pack_core.h
// (shared with the window flush of the decode kernel).
//
// One workgroup (256 threads, 4 waves) owns one block of one (batch, kv
// head) unit: it stages the 32 x 128 key and value tiles in LDS with 16-byte
// coalesced loads, reduces the group minima/maxima, then writes whole 32-bit
// code words with coalesced stores.  Extra workgroups of the same launch copy
// the trailing tokens into the residual window.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kivi_internal.h"
#include "kivi_pack_core.h"

namespace kivi {
namespace {

using namespace packcore;
constexpr int kCopy = 32;  // window tokens copied per workgroup

// TF: how near ties are repaired (Tie::kMask or Tie::kDev, see code_of).
template <int KB, int VB, bool BF16, int G, Tie TF>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  __shared__ __align__(16) uint8_t lds[PackLds<G>::bytes];
  const int tid = threadIdx.x;
  const int item = blockIdx.x;
  // this unit's work: the launch's, or its sequence's in a ragged launch
  long long u = blockIdx.y;
  int nblk = a.nblk, src_tok0 = a.src_tok0, dst_blk0 = a.dst_blk0;
  int r_src_tok0 = a.r_src_tok0, r_count = a.r_count, r_dst_slot0 = a.r_dst_slot0;
  if (a.ragged) {
    const SeqOp& o = a.op[blockIdx.y / a.H];
    u = a.unit0 + (long long)blockIdx.y;
    nblk = o.nblk;
    src_tok0 = o.src_tok0;
    dst_blk0 = o.dst_blk0;
    r_src_tok0 = o.r_src_tok0;
    r_count = o.r_count;
    r_dst_slot0 = o.r_dst_slot0;
    if (item >= nblk + (r_count + kCopy - 1) / kCopy) return;  // the grid covers the longest sequence
  }

  if (item >= nblk) {
    // ---- residual-window copy: 32 tokens per workgroup
    const int t0 = (item - nblk) * kCopy;
    const int n = min(kCopy, r_count - t0);
    for (int c = tid; c < n * (D / 8); c += 256) {
      const int t = t0 + c / (D / 8), col = (c % (D / 8)) * 8;
      const long long src = u * a.r_src_unit_stride + (long long)(r_src_tok0 + t) * D + col;
      const long long dst = (u * a.R + r_dst_slot0 + t) * D + col;
      *reinterpret_cast<uint4*>(a.k_resid + dst) = *reinterpret_cast<const uint4*>(a.rk_src + src);
      *reinterpret_cast<uint4*>(a.v_resid + dst) = *reinterpret_cast<const uint4*>(a.rv_src + src);
    }
    return;
  }

  // ---- quantize and pack block `item` of this unit
  constexpr BlockLayout BL = block_layout(KB, VB, G);
  const long long ri = record_index(a.page_table, a.page_stride, a.num_pages, a.nb, a.H, u, dst_blk0 + item);
  const long long src = u * a.src_unit_stride + (long long)(src_tok0 + item * G) * D;
  pack_block<KB, VB, BF16, G, TF, 256>(a.k_src + src, a.v_src + src, a.blocks + ri * BL.bytes, a.scale_max + ri, lds,
                                       tid);
}

template <int KB, int VB, bool BF16>
hipError_t launch_pack_t(const PackArgs& a, hipStream_t stream) {
  int items = a.nblk + (a.r_count + kCopy - 1) / kCopy;
  if (a.ragged) {  // a.units units of a.units / a.H sequences: the longest sets the grid
    items = 0;
    for (int i = 0; i < a.units / a.H; ++i)
      items = max(items, a.op[i].nblk + (a.op[i].r_count + kCopy - 1) / kCopy);
  }
  if (items == 0 || a.units == 0) return hipSuccess;
  dim3 grid(items, a.units);
  // The tie repair by mask costs registers (fewer resident workgroups) and
  // saves vector work: it pays for bf16 inputs (frequent ties) and for
  // launches of at most one round of workgroups (a window flush), whose time
  // is one workgroup's latency; big fp16 launches are bound by memory and
  // keep the careful pass.  64-token blocks keep it too.
  const bool one_round = (long long)items * a.units <= 256LL * 8;
  if (a.G == 64) {
    hipLaunchKernelGGL((pack_kernel<KB, VB, BF16, 64, Tie::kDev>), grid, dim3(256), 0, stream, a);
  } else if (BF16 || one_round) {
    hipLaunchKernelGGL((pack_kernel<KB, VB, BF16, 32, Tie::kMask>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((pack_kernel<KB, VB, BF16, 32, Tie::kDev>), grid, dim3(256), 0, stream, a);
  }
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
