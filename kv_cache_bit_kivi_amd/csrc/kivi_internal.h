// kivi_internal.h - argument blocks and kernel launchers shared by the host
// state machine (kivi_api.cpp) and the HIP kernels (*.hip).  Not installed.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kivi {

constexpr int kGroup = 32;       // default G: tokens per key group, channels per value group
constexpr int kStream = 32;      // decode: tokens per stream (a group, or half of a 64-token group)
constexpr int kHeadDim = 128;    // D handled by the kernels
constexpr int kMaxSplits = 256;  // upper bound on decode token splits

// Byte offsets of the fields of one packed block record (one unit, G
// tokens) and its size; the layout is documented in include/kivi.h.
struct BlockLayout {
  int k_codes, v_codes, k_scale, k_zero, v_scale, v_zero, bytes;
};
__host__ __device__ constexpr BlockLayout block_layout(int k_bits, int v_bits, int g = kGroup) {
  return BlockLayout{0,
                     g * kHeadDim * k_bits / 8,
                     g * kHeadDim * (k_bits + v_bits) / 8,
                     g * kHeadDim * (k_bits + v_bits) / 8 + 2 * kHeadDim,
                     g * kHeadDim * (k_bits + v_bits) / 8 + 4 * kHeadDim,
                     g * kHeadDim * (k_bits + v_bits) / 8 + 6 * kHeadDim,
                     g * kHeadDim * (k_bits + v_bits) / 8 + 8 * kHeadDim};
}

// Paged block records (page_table != nullptr): block g of sequence b, kv
// head h lives at blocks + (P * H + h) * block_bytes with page
// P = page_table[b * page_stride + g], clamped into [0, num_pages) so that a
// wrong table can never address memory outside the pool.
__host__ __device__ inline long long record_index(const int32_t* page_table, int page_stride, int num_pages,
                                                 int nb, int H, long long u, int g) {
  if (!page_table) return u * nb + g;
  const long long b = u / H;
  int p = page_table[b * page_stride + g];
  p = p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
  return (long long)p * H + (u - b * H);
}

// Per-sequence work of a pack launch over sequences of different lengths
// (same fields as the uniform ones of PackArgs).
struct SeqOp {
  int src_tok0, nblk, dst_blk0, r_src_tok0, r_count, r_dst_slot0;
};
constexpr int kPackChunk = 32;    // sequences per ragged pack launch
constexpr int kDecodeChunk = 64;  // sequences per ragged decode launch

// One launch of the pack kernel: quantize + bit-pack `nblk` blocks of G
// tokens per unit, and copy `r_count` tokens per unit into the window.
// Ragged launches (ragged != 0) cover units unit0 .. unit0 + gridDim.y - 1,
// H per sequence, and take each sequence's work from op[] instead.
struct PackArgs {
  // tokens to pack: unit u, token i is at src + u * src_unit_stride + i * D
  const uint16_t* k_src;
  const uint16_t* v_src;
  long long src_unit_stride;  // elements
  int src_tok0;               // first source token to pack
  int nblk;                   // blocks of G tokens to pack per unit
  int dst_blk0;               // destination block index (n_quant / G)
  // tokens to copy into the residual window (0 when r_count == 0)
  const uint16_t* rk_src;
  const uint16_t* rv_src;
  long long r_src_unit_stride;
  int r_src_tok0;
  int r_count;
  int r_dst_slot0;
  // cache arrays
  uint8_t* blocks;  // [units][nb] block records
  // per block record (same index as the record): the largest stored key
  // scale (fp16 bits, low half) and value scale (high half) of the record
  uint32_t* scale_max;
  uint16_t* k_resid;
  uint16_t* v_resid;
  int cap;    // token capacity per unit
  int nb;     // blocks per unit (cap / G)
  int R;      // window length
  int units;  // B * H
  int G;      // tokens per block (32 or 64)
  const int32_t* page_table;  // paged block records (nullptr: unit-major)
  int page_stride, num_pages;
  int ragged;
  int unit0;  // ragged: first unit of the launch (a sequence boundary)
  int H;      // ragged: units per sequence
  SeqOp op[kPackChunk];
};

// One decode-attention launch (split kernel + merge kernel).
struct DecodeArgs {
  const uint8_t* blocks;  // [B*H][nb] block records
  const uint32_t* scale_max;  // per record: largest key scale | largest value scale << 16
  const uint16_t* k_resid;
  const uint16_t* v_resid;
  const uint16_t* q;   // [B][Hq][D] kv dtype
  void* out;           // [B][Hq][D] out dtype
  float* partial;      // [B][Hq][n_split][D + 2] fp32 (m, l, o[D])
  int B, H, Hq, gq;
  int cap, nb, R;
  int G;  // tokens per block (32 or 64); the kernels work in 32-token streams
  const int32_t* page_table;  // paged block records (nullptr: unit-major)
  int page_stride, num_pages;
  int n_quant, n_resid;
  int n_split;
  int n_split_packed;   // splits over packed groups (the window split follows)
  int groups_per_split; // packed groups per split, a multiple of 4
  int hg;               // workgroups per (unit, split): query heads per kv head / 4 above 4, else 1
  float qscale;         // softmax_scale * log2(e): scores in base-2 units
  // ragged launches (ragged != 0) cover sequences seq0 .. seq0 + gridDim.y / H
  // - 1 and take each one's lengths from seq_len[][2] = (n_quant, n_resid);
  // n_quant and n_resid above are then the largest of the whole cache
  int ragged;
  int seq0;
  int seq_len[kDecodeChunk][2];
  // fused append (k_new != nullptr): each unit's newest window token, slot
  // n_resid - 1, is read from k_new / v_new ([B][H][D]) and stored into the
  // window by the wave that runs the window (of the first head group)
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_resid_w;  // the window arrays, writable (fused append)
  uint16_t* v_resid_w;
};

// LDS bytes of one workgroup (key wave + value wave) of the matrix-core
// decode kernel serving `heads` query heads (4, or 8 in the eight-head
// layout): one key-code buffer, two key-metadata buffers, two value stages
// and two hand-over buffers.  Bounds the resident workgroups per CU.
constexpr int mfma_wg_lds_bytes(int k_bits, int v_bits, int heads) {
  return 4 * (kGroup * kHeadDim * k_bits / 8 + 64) + 2 * (2 * 4 * kHeadDim * 2) +
         2 * (4 * kGroup * v_bits / 32 * kHeadDim * 4 + 2 * 4 * kHeadDim * 2) +
         2 * (4 * heads * 36 * 4 + 4 * heads + 16 * heads);
}
constexpr int kLdsPerCu = 160 * 1024;  // MI355X (gfx950)

// dtype codes: 0 fp16, 1 bf16, 2 fp32 (matches kivi_dtype)
hipError_t launch_pack(const PackArgs& a, int k_bits, int v_bits, int kv_dtype,
                       hipStream_t stream);
hipError_t launch_resid_copy(const PackArgs& a, int kv_dtype, hipStream_t stream);
// Split kernel (matrix cores, 1, 2, 4, 8 or 16 query heads per kv head),
// then the merge.  split_begin / split_end (may be null): events recorded on
// the stream right before and right after the split kernel.
hipError_t launch_decode(const DecodeArgs& a, int k_bits, int v_bits, int kv_dtype,
                         int out_dtype, hipStream_t stream,
                         hipEvent_t split_begin, hipEvent_t split_end);
hipError_t launch_decode_mfma(const DecodeArgs& a, int k_bits, int v_bits, int kv_dtype,
                                  hipStream_t stream);
// Streaming read of `bytes` (a multiple of 16) from src by `workgroups`
// workgroups of 256 threads; each thread writes one word of its XOR to sink.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t stream);

}  // namespace kivi

#include "../../include/kivi.h"

namespace kivi {
// Decode attention over the cache's current state with the partials in
// `scratch` (scratch_bytes long): the entry point without a workspace
// argument checks the planned partials, not the worst case, against its
// fixed array.  Same kernels and plan as kivi_decode_attn.
kivi_status decode_attn_bounded(kivi_cache* cache, const void* q, int32_t num_q_heads, float softmax_scale,
                                void* out, int32_t out_dtype, void* scratch, size_t scratch_bytes,
                                void* stream);
// Returns `s` and sets the thread's kivi_last_error_message() text.
kivi_status report(kivi_status s, const char* message);
}  // namespace kivi
