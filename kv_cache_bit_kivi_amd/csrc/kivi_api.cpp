// kivi_api.cpp - host state machine and C ABI (include/kivi.h).
//
// The cache is one attention layer: packed codes and metadata for tokens
// [0, n_quant) plus an unquantized residual window for [n_quant, T).  The
// window policy follows page "KIVI: Asymmetric 2-Bit KV Cache Quantization
// Guide", item 3 of "The Three Structural Innovations of KIVI" and "Step 3":
// new tokens enter the full-precision window, and a full window is grouped
// and packed before the next token enters (whole-window flush, so the window
// holds 1..R tokens after any append).  Appending n tokens at once produces
// exactly the state of n single appends; full windows inside the input are
// packed straight from the caller's buffer.
//
// Every entry point validates its arguments before enqueuing anything; the
// counters advance at enqueue time.  A failed launch poisons the handle.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/kivi.h"
#include "kivi_internal.h"

struct kivi_cache {
  kivi_config cfg;
  int cap;  // token capacity per unit (max_tokens rounded up to R)
  int nb;   // blocks per unit
  int n_quant;  // every sequence's, or the largest when ragged
  int n_resid;
  // sequences of different lengths (per-sequence appends or resets): the
  // per-sequence counters below are then the state
  bool ragged;
  std::vector<int> sq, sr;  // n_quant, n_resid of each sequence (ragged)
  // paged block records (kivi_cache_set_page_table); nullptr: unit-major
  const int32_t* page_table;
  int page_stride, num_pages;
  int forced_splits;
  int cu_count;  // compute units of the device (0: not known yet)
  bool poisoned;
  // measurement: events recorded around each split-kernel launch (or null)
  hipEvent_t ev_split_begin, ev_split_end;
  uint8_t* blocks;  // [B*H][nb] block records
  uint32_t* scale_max;  // one entry per block record (same index)
  uint16_t* k_resid;
  uint16_t* v_resid;
  // The last decode plan and the inputs it was made from.  The ragged plan
  // search loops over split sizes and sequences; its inputs (the packed
  // lengths) change once every R tokens of a sequence, so most decode steps
  // reuse the plan.  Only plan_decode reads or writes these.
  mutable bool memo_valid;
  mutable int memo_key[6];
  mutable std::vector<int> memo_sq;
  mutable int memo_plan[4];
};

namespace {

thread_local std::string g_last_error;

kivi_status fail(kivi_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kivi_status fail(kivi_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t off[4];  // blocks, k_resid, v_resid, scale_max
  size_t total;
  int cap, nb;
};

kivi_status check_config(const kivi_config* c) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "config is NULL");
  if (c->batch < 1 || c->num_kv_heads < 1 || c->head_dim < 1 || c->max_tokens < 1)
    return fail(KIVI_ERR_INVALID_ARG, "batch, num_kv_heads, head_dim and max_tokens must be >= 1");
  if ((c->k_bits != 2 && c->k_bits != 4) || (c->v_bits != 2 && c->v_bits != 4))
    return fail(KIVI_ERR_INVALID_ARG, "k_bits and v_bits must be 2 or 4 (got %d, %d)", c->k_bits,
                c->v_bits);
  if (c->group_size < 2 || c->head_dim % c->group_size != 0)
    return fail(KIVI_ERR_INVALID_ARG, "head_dim (%d) must be a multiple of group_size (%d)",
                c->head_dim, c->group_size);
  if (c->residual_length < c->group_size || c->residual_length % c->group_size != 0 ||
      c->residual_length > 1024)
    return fail(KIVI_ERR_INVALID_ARG,
                "residual_length (%d) must be a positive multiple of group_size, at most 1024",
                c->residual_length);
  if (c->kv_dtype != KIVI_F16 && c->kv_dtype != KIVI_BF16)
    return fail(KIVI_ERR_INVALID_ARG, "kv_dtype must be KIVI_F16 or KIVI_BF16");
  if (c->head_dim != kivi::kHeadDim || (c->group_size != 32 && c->group_size != 64))
    return fail(KIVI_ERR_UNSUPPORTED, "kernels are built for head_dim %d and group_size 32 or 64",
                kivi::kHeadDim);
  if ((long long)c->batch * c->num_kv_heads > 65535)
    return fail(KIVI_ERR_UNSUPPORTED, "batch * num_kv_heads must be at most 65535");
  if ((long long)c->max_tokens + c->residual_length > (1LL << 30))
    return fail(KIVI_ERR_UNSUPPORTED, "max_tokens too large");
  return KIVI_OK;
}

Layout layout_of(const kivi_config* c) {
  Layout L;
  const size_t U = (size_t)c->batch * c->num_kv_heads;
  const size_t D = c->head_dim, G = c->group_size, R = c->residual_length;
  L.cap = (int)(((size_t)c->max_tokens + R - 1) / R * R);
  L.nb = (int)(L.cap / G);
  const size_t block_bytes = G * D * (c->k_bits + c->v_bits) / 8 + 8 * D;
  const size_t sizes[4] = {
      U * L.nb * block_bytes,  // block records
      U * R * D * 2,           // k_resid
      U * R * D * 2,           // v_resid
      U * L.nb * 4,            // scale_max: one u32 per block record
  };
  size_t o = 0;
  for (int i = 0; i < 4; ++i) {
    L.off[i] = o;
    o = align_up(o + sizes[i]);
  }
  L.total = o;
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kivi::PackArgs base_pack_args(const kivi_cache* c) {
  kivi::PackArgs a{};
  a.blocks = c->blocks;
  a.scale_max = c->scale_max;
  a.k_resid = c->k_resid;
  a.v_resid = c->v_resid;
  a.cap = c->cap;
  a.nb = c->nb;
  a.R = c->cfg.residual_length;
  a.units = c->cfg.batch * c->cfg.num_kv_heads;
  a.G = c->cfg.group_size;
  a.H = c->cfg.num_kv_heads;
  a.page_table = c->page_table;
  a.page_stride = c->page_stride;
  a.num_pages = c->num_pages;
  return a;
}

kivi_status hip_fail(kivi_cache* c, hipError_t e, const char* what) {
  if (c) c->poisoned = true;
  return fail(KIVI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Packs the full window (R tokens) into positions n_quant .. n_quant + R - 1.
kivi_status flush_window(kivi_cache* c, hipStream_t s) {
  kivi::PackArgs a = base_pack_args(c);
  const int R = c->cfg.residual_length, D = c->cfg.head_dim;
  a.k_src = c->k_resid;
  a.v_src = c->v_resid;
  a.src_unit_stride = (long long)R * D;
  a.src_tok0 = 0;
  a.nblk = R / c->cfg.group_size;
  a.dst_blk0 = c->n_quant / c->cfg.group_size;
  a.r_count = 0;
  hipError_t e = kivi::launch_pack(a, c->cfg.k_bits, c->cfg.v_bits, c->cfg.kv_dtype, s);
  if (e != hipSuccess) return hip_fail(c, e, "pack (window flush) launch");
  c->n_quant += R;
  c->n_resid = 0;
  return KIVI_OK;
}

// Copies input tokens [tok0, tok0 + n) of every unit into window slots
// [n_resid, n_resid + n).
kivi_status copy_to_window(kivi_cache* c, const uint16_t* k, const uint16_t* v,
                           long long unit_stride, int tok0, int n, hipStream_t s) {
  kivi::PackArgs a = base_pack_args(c);
  a.rk_src = k;
  a.rv_src = v;
  a.r_src_unit_stride = unit_stride;
  a.r_src_tok0 = tok0;
  a.r_count = n;
  a.r_dst_slot0 = c->n_resid;
  hipError_t e = kivi::launch_resid_copy(a, c->cfg.kv_dtype, s);
  if (e != hipSuccess) return hip_fail(c, e, "window copy launch");
  c->n_resid += n;
  return KIVI_OK;
}

// ---- sequences of different lengths
//
// Each sequence follows the single-sequence rules above.  A ragged append
// runs in up to four phases, each one pack launch per chunk of kPackChunk
// sequences with per-sequence work: (A) pack the full windows of sequences
// receiving tokens, (B) top up windows that the new tokens overflow, (C) pack
// those, (D) pack whole windows straight from the input and copy the rest
// into the window.

void make_ragged(kivi_cache* c) {
  if (c->ragged) return;
  c->sq.assign(c->cfg.batch, c->n_quant);
  c->sr.assign(c->cfg.batch, c->n_resid);
  c->ragged = true;
}

// Back to the uniform representation when every sequence has the same
// lengths; otherwise n_quant / n_resid become the largest ones.
void settle(kivi_cache* c) {
  if (!c->ragged) return;
  bool same = true;
  int mq = 0, mr = 0;
  for (int b = 0; b < c->cfg.batch; ++b) {
    same = same && c->sq[b] == c->sq[0] && c->sr[b] == c->sr[0];
    mq = std::max(mq, c->sq[b]);
    mr = std::max(mr, c->sr[b]);
  }
  c->n_quant = mq;
  c->n_resid = mr;
  if (same) c->ragged = false;
}

// One ragged pack phase: ops[b] for every sequence (empty ops do nothing).
kivi_status launch_ragged_phase(kivi_cache* c, const std::vector<kivi::SeqOp>& ops,
                                const uint16_t* k_src, const uint16_t* v_src, long long src_stride,
                                const uint16_t* rk_src, const uint16_t* rv_src, long long r_stride,
                                hipStream_t s) {
  const int B = c->cfg.batch, H = c->cfg.num_kv_heads;
  for (int b0 = 0; b0 < B; b0 += kivi::kPackChunk) {
    const int nseq = std::min(kivi::kPackChunk, B - b0);
    bool any = false;
    kivi::PackArgs a = base_pack_args(c);
    a.ragged = 1;
    a.unit0 = b0 * H;
    a.H = H;
    a.units = nseq * H;
    a.k_src = k_src;
    a.v_src = v_src;
    a.src_unit_stride = src_stride;
    a.rk_src = rk_src;
    a.rv_src = rv_src;
    a.r_src_unit_stride = r_stride;
    for (int i = 0; i < nseq; ++i) {
      a.op[i] = ops[b0 + i];
      any = any || a.op[i].nblk > 0 || a.op[i].r_count > 0;
    }
    if (!any) continue;
    hipError_t e = kivi::launch_pack(a, c->cfg.k_bits, c->cfg.v_bits, c->cfg.kv_dtype, s);
    if (e != hipSuccess) return hip_fail(c, e, "pack launch (sequences of different lengths)");
  }
  return KIVI_OK;
}

// Packs the full window of every sequence with flush[b] set.
kivi_status ragged_flush(kivi_cache* c, const std::vector<char>& flush, hipStream_t s) {
  const int B = c->cfg.batch, R = c->cfg.residual_length, G = c->cfg.group_size;
  std::vector<kivi::SeqOp> ops(B, kivi::SeqOp{0, 0, 0, 0, 0, 0});
  bool any = false;
  for (int b = 0; b < B; ++b) {
    if (!flush[b]) continue;
    ops[b].nblk = R / G;
    ops[b].dst_blk0 = c->sq[b] / G;
    any = true;
  }
  if (!any) return KIVI_OK;
  const long long stride = (long long)R * c->cfg.head_dim;
  kivi_status st = launch_ragged_phase(c, ops, c->k_resid, c->v_resid, stride, nullptr, nullptr, 0, s);
  if (st != KIVI_OK) return st;
  for (int b = 0; b < B; ++b) {
    if (!flush[b]) continue;
    c->sq[b] += R;
    c->sr[b] = 0;
  }
  return KIVI_OK;
}

// Appends n[b] tokens to sequence b from k, v laid out [B][H][n_max][D].
kivi_status ragged_append(kivi_cache* c, const uint16_t* k, const uint16_t* v, const int32_t* n,
                          int n_max, hipStream_t s) {
  const int B = c->cfg.batch, R = c->cfg.residual_length, G = c->cfg.group_size;
  const long long stride = (long long)n_max * c->cfg.head_dim;
  make_ragged(c);
  kivi_status st;
  // (A) a full window is packed before the next token enters it
  std::vector<char> fl(B, 0);
  for (int b = 0; b < B; ++b) fl[b] = n[b] > 0 && c->sr[b] == R;
  if ((st = ragged_flush(c, fl, s)) != KIVI_OK) return st;
  // (B) top up windows the new tokens overflow, (C) pack them
  std::vector<int> pos(B, 0);
  std::vector<kivi::SeqOp> ops(B, kivi::SeqOp{0, 0, 0, 0, 0, 0});
  bool any = false;
  for (int b = 0; b < B; ++b) {
    fl[b] = c->sr[b] > 0 && c->sr[b] + n[b] > R;
    if (!fl[b]) continue;
    pos[b] = R - c->sr[b];
    ops[b].r_count = pos[b];
    ops[b].r_dst_slot0 = c->sr[b];
    any = true;
  }
  if (any) {
    if ((st = launch_ragged_phase(c, ops, nullptr, nullptr, 0, k, v, stride, s)) != KIVI_OK) return st;
    for (int b = 0; b < B; ++b)
      if (fl[b]) c->sr[b] = R;
    if ((st = ragged_flush(c, fl, s)) != KIVI_OK) return st;
  }
  // (D) the rest: whole windows straight from the input, the last 1..R
  // tokens into an empty window; or everything into a partly filled window
  std::vector<int> nq2(c->sq), nr2(c->sr);
  any = false;
  for (int b = 0; b < B; ++b) {
    ops[b] = kivi::SeqOp{0, 0, 0, 0, 0, 0};
    const int rem = n[b] - pos[b];
    if (rem <= 0) continue;
    any = true;
    if (c->sr[b] == 0) {
      const int keep = (rem - 1) % R + 1;
      const int npack = rem - keep;
      ops[b] = kivi::SeqOp{pos[b], npack / G, c->sq[b] / G, pos[b] + npack, keep, 0};
      nq2[b] += npack;
      nr2[b] = keep;
    } else {
      ops[b] = kivi::SeqOp{0, 0, 0, pos[b], rem, c->sr[b]};
      nr2[b] += rem;
    }
  }
  if (any) {
    if ((st = launch_ragged_phase(c, ops, k, v, stride, k, v, stride, s)) != KIVI_OK) return st;
    c->sq = nq2;
    c->sr = nr2;
  }
  settle(c);
  return KIVI_OK;
}

size_t workspace_bytes_for(const kivi_cache* c, int hq, int n_split) {
  return (size_t)c->cfg.batch * hq * n_split * (c->cfg.head_dim + 2) * sizeof(float);
}

// Largest split count a decode launch can use: the kernels split the token
// axis into 32-token streams (a block of G = 32, or half a block of G = 64),
// the packed ones plus the window's.
int max_items(const kivi_cache* c) {
  return c->cap / kivi::kStream + c->cfg.residual_length / kivi::kStream;
}

}  // namespace

extern "C" {

kivi_status kivi_cache_bytes(const kivi_config* cfg, size_t* bytes) {
  kivi_status s = check_config(cfg);
  if (s != KIVI_OK) return s;
  if (!bytes) return fail(KIVI_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout_of(cfg).total;
  return KIVI_OK;
}

kivi_status kivi_cache_create(const kivi_config* cfg, void* dev_buf, size_t dev_bytes,
                              kivi_cache** out) {
  kivi_status s = check_config(cfg);
  if (s != KIVI_OK) return s;
  if (!dev_buf || !out) return fail(KIVI_ERR_INVALID_ARG, "dev_buf and out must not be NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) % kAlign)
    return fail(KIVI_ERR_INVALID_ARG, "dev_buf must be 256-byte aligned");
  const Layout L = layout_of(cfg);
  if (dev_bytes < L.total)
    return fail(KIVI_ERR_BUFFER_TOO_SMALL, "cache needs %zu bytes, got %zu", L.total, dev_bytes);
  kivi_cache* c = new (std::nothrow) kivi_cache();
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "host allocation failed");
  c->cfg = *cfg;
  c->cap = L.cap;
  c->nb = L.nb;
  char* base = static_cast<char*>(dev_buf);
  c->blocks = reinterpret_cast<uint8_t*>(base + L.off[0]);
  c->k_resid = reinterpret_cast<uint16_t*>(base + L.off[1]);
  c->v_resid = reinterpret_cast<uint16_t*>(base + L.off[2]);
  c->scale_max = reinterpret_cast<uint32_t*>(base + L.off[3]);
  // the decode's split planner needs the compute-unit count; a failed
  // query is repeated by the first decode call
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    c->cu_count = cus;
  *out = c;
  return KIVI_OK;
}

kivi_status kivi_cache_destroy(kivi_cache* cache) {
  delete cache;
  return KIVI_OK;
}

kivi_status kivi_cache_reset(kivi_cache* cache) {
  if (!cache) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (cache->poisoned) return fail(KIVI_ERR_HIP, "cache handle is poisoned by an earlier HIP error");
  cache->n_quant = 0;
  cache->n_resid = 0;
  cache->ragged = false;
  return KIVI_OK;
}

kivi_status kivi_cache_reset_sequences(kivi_cache* c, const int32_t* seqs, int32_t count) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (c->poisoned) return fail(KIVI_ERR_HIP, "cache handle is poisoned by an earlier HIP error");
  if (count < 0 || (count > 0 && !seqs)) return fail(KIVI_ERR_INVALID_ARG, "bad sequence list");
  for (int i = 0; i < count; ++i)
    if (seqs[i] < 0 || seqs[i] >= c->cfg.batch)
      return fail(KIVI_ERR_INVALID_ARG, "sequence %d out of range [0, %d)", seqs[i], c->cfg.batch);
  if (count == 0) return KIVI_OK;
  make_ragged(c);
  for (int i = 0; i < count; ++i) c->sq[seqs[i]] = c->sr[seqs[i]] = 0;
  settle(c);
  return KIVI_OK;
}

kivi_status kivi_cache_set_page_table(kivi_cache* c, const int32_t* table, int32_t page_stride,
                                      int32_t num_pages) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (!table) {
    c->page_table = nullptr;
    c->page_stride = c->num_pages = 0;
    return KIVI_OK;
  }
  if (reinterpret_cast<uintptr_t>(table) % 4) return fail(KIVI_ERR_INVALID_ARG, "table must be 4-byte aligned");
  if (page_stride < c->nb)
    return fail(KIVI_ERR_INVALID_ARG, "page_stride (%d) must cover the %d blocks of a sequence", page_stride, c->nb);
  if (num_pages < 1 || (long long)num_pages > (long long)c->cfg.batch * c->nb)
    return fail(KIVI_ERR_INVALID_ARG, "num_pages (%d) must be in [1, batch * blocks = %lld]", num_pages,
                (long long)c->cfg.batch * c->nb);
  c->page_table = table;
  c->page_stride = page_stride;
  c->num_pages = num_pages;
  return KIVI_OK;
}

kivi_status kivi_cache_get_lengths(const kivi_cache* c, int32_t* n_quant, int32_t* n_resid) {
  if (!c || !n_quant || !n_resid) return fail(KIVI_ERR_INVALID_ARG, "cache and outputs must not be NULL");
  for (int b = 0; b < c->cfg.batch; ++b) {
    n_quant[b] = c->ragged ? c->sq[b] : c->n_quant;
    n_resid[b] = c->ragged ? c->sr[b] : c->n_resid;
  }
  return KIVI_OK;
}

kivi_status kivi_append(kivi_cache* c, const void* k, const void* v, int32_t n_tokens,
                        void* stream) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (c->poisoned) return fail(KIVI_ERR_HIP, "cache handle is poisoned by an earlier HIP error");
  if (n_tokens < 0) return fail(KIVI_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens == 0) return KIVI_OK;
  if (!k || !v) return fail(KIVI_ERR_INVALID_ARG, "k and v must not be NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(KIVI_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  int longest = c->n_quant + c->n_resid;
  if (c->ragged) {
    longest = 0;
    for (int b = 0; b < c->cfg.batch; ++b) longest = std::max(longest, c->sq[b] + c->sr[b]);
  }
  if ((long long)longest + n_tokens > c->cfg.max_tokens)
    return fail(KIVI_ERR_CAPACITY, "appending %d tokens to %d exceeds max_tokens %d", n_tokens,
                longest, c->cfg.max_tokens);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  if (c->ragged) {  // every sequence takes n_tokens, each from its own state
    const std::vector<int32_t> n(c->cfg.batch, n_tokens);
    return ragged_append(c, kk, vv, n.data(), n_tokens, s);
  }
  const int R = c->cfg.residual_length, G = c->cfg.group_size, D = c->cfg.head_dim;
  const long long stride = (long long)n_tokens * D;
  kivi_status st;

  // A full window is packed before the next token enters it.
  if (c->n_resid == R) {
    if ((st = flush_window(c, s)) != KIVI_OK) return st;
  }
  int pos = 0;
  if (c->n_resid > 0 && c->n_resid + n_tokens > R) {
    // top the window up, then pack it: more tokens follow
    const int fill = R - c->n_resid;
    if ((st = copy_to_window(c, kk, vv, stride, 0, fill, s)) != KIVI_OK) return st;
    if ((st = flush_window(c, s)) != KIVI_OK) return st;
    pos = fill;
  }
  const int rem = n_tokens - pos;
  if (c->n_resid == 0) {
    // empty window: every full window but the last goes straight to the
    // packed store; the last 1..R tokens enter the window (same launch)
    const int keep = (rem - 1) % R + 1;
    const int npack = rem - keep;
    kivi::PackArgs a = base_pack_args(c);
    a.k_src = kk;
    a.v_src = vv;
    a.src_unit_stride = stride;
    a.src_tok0 = pos;
    a.nblk = npack / G;
    a.dst_blk0 = c->n_quant / G;
    a.rk_src = kk;
    a.rv_src = vv;
    a.r_src_unit_stride = stride;
    a.r_src_tok0 = pos + npack;
    a.r_count = keep;
    a.r_dst_slot0 = 0;
    hipError_t e = kivi::launch_pack(a, c->cfg.k_bits, c->cfg.v_bits, c->cfg.kv_dtype, s);
    if (e != hipSuccess) return hip_fail(c, e, "pack launch");
    c->n_quant += npack;
    c->n_resid = keep;
  } else {
    if ((st = copy_to_window(c, kk, vv, stride, pos, rem, s)) != KIVI_OK) return st;
  }
  return KIVI_OK;
}

kivi_status kivi_append_varlen(kivi_cache* c, const void* k, const void* v, const int32_t* n_tokens,
                               int32_t n_max, void* stream) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (c->poisoned) return fail(KIVI_ERR_HIP, "cache handle is poisoned by an earlier HIP error");
  if (!n_tokens) return fail(KIVI_ERR_INVALID_ARG, "n_tokens is NULL");
  if (n_max < 0) return fail(KIVI_ERR_INVALID_ARG, "n_max must be >= 0");
  const int B = c->cfg.batch;
  bool any = false, all_max = true;
  for (int b = 0; b < B; ++b) {
    if (n_tokens[b] < 0 || n_tokens[b] > n_max)
      return fail(KIVI_ERR_INVALID_ARG, "n_tokens[%d] = %d is outside [0, n_max = %d]", b, n_tokens[b], n_max);
    any = any || n_tokens[b] > 0;
    all_max = all_max && n_tokens[b] == n_max;
  }
  if (!any) return KIVI_OK;
  if (!k || !v) return fail(KIVI_ERR_INVALID_ARG, "k and v must not be NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(KIVI_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  for (int b = 0; b < B; ++b) {
    const int t = c->ragged ? c->sq[b] + c->sr[b] : c->n_quant + c->n_resid;
    if ((long long)t + n_tokens[b] > c->cfg.max_tokens)
      return fail(KIVI_ERR_CAPACITY, "sequence %d: appending %d tokens to %d exceeds max_tokens %d", b,
                  n_tokens[b], t, c->cfg.max_tokens);
  }
  if (all_max && !c->ragged) return kivi_append(c, k, v, n_max, stream);
  return ragged_append(c, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), n_tokens,
                       n_max, static_cast<hipStream_t>(stream));
}

kivi_status kivi_flush_residual(kivi_cache* c, void* stream) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (c->poisoned) return fail(KIVI_ERR_HIP, "cache handle is poisoned by an earlier HIP error");
  if (c->ragged) {
    std::vector<char> fl(c->cfg.batch, 0);
    for (int b = 0; b < c->cfg.batch; ++b) fl[b] = c->sr[b] == c->cfg.residual_length;
    kivi_status st = ragged_flush(c, fl, static_cast<hipStream_t>(stream));
    if (st == KIVI_OK) settle(c);
    return st;
  }
  if (c->n_resid != c->cfg.residual_length) return KIVI_OK;
  return flush_window(c, static_cast<hipStream_t>(stream));
}

kivi_status kivi_decode_attn_workspace_bytes(const kivi_cache* c, int32_t num_q_heads,
                                             size_t* bytes) {
  if (!c || !bytes) return fail(KIVI_ERR_INVALID_ARG, "cache and bytes must not be NULL");
  if (num_q_heads < 1 || num_q_heads % c->cfg.num_kv_heads)
    return fail(KIVI_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, c->cfg.num_kv_heads);
  *bytes = workspace_bytes_for(c, num_q_heads, std::min(kivi::kMaxSplits, max_items(c)));
  return KIVI_OK;
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points (the cache may still be empty:
// the fused append adds a token first).
kivi_status check_decode_args(const kivi_cache* c, const void* q, int32_t num_q_heads, void* out,
                              int32_t out_dtype, void* workspace, size_t ws_bytes) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (c->poisoned) return fail(KIVI_ERR_HIP, "cache handle is poisoned by an earlier HIP error");
  if (!q || !out || !workspace) return fail(KIVI_ERR_INVALID_ARG, "q, out and workspace must not be NULL");
  if (num_q_heads < 1 || num_q_heads % c->cfg.num_kv_heads)
    return fail(KIVI_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, c->cfg.num_kv_heads);
  if (out_dtype != KIVI_F16 && out_dtype != KIVI_BF16 && out_dtype != KIVI_F32)
    return fail(KIVI_ERR_INVALID_ARG, "bad out_dtype %d", out_dtype);
  const int gq = num_q_heads / c->cfg.num_kv_heads;
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8 && gq != 16)
    return fail(KIVI_ERR_UNSUPPORTED, "query heads per kv head must be 1, 2, 4, 8 or 16 (got %d)", gq);
  size_t need = 0;
  kivi_decode_attn_workspace_bytes(c, num_q_heads, &need);
  if (ws_bytes < need)
    return fail(KIVI_ERR_BUFFER_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  return KIVI_OK;
}

// Lengths of every sequence: the cache's, or the state a decode step will
// see after its token append.
struct DecodeState {
  bool ragged;
  int n_quant, n_resid;     // every sequence's, or the largest (ragged)
  std::vector<int> sq, sr;  // per sequence (ragged)
};

DecodeState state_of(const kivi_cache* c) {
  DecodeState st{c->ragged, c->n_quant, c->n_resid, {}, {}};
  if (c->ragged) {
    st.sq = c->sq;
    st.sr = c->sr;
  }
  return st;
}

// The state after one token per sequence: a full window is packed first
// (n_quant += R, n_resid = 0), then the token enters the window.
DecodeState after_token(const kivi_cache* c) {
  const int R = c->cfg.residual_length;
  DecodeState st = state_of(c);
  if (!st.ragged) {
    if (st.n_resid == R) {
      st.n_quant += R;
      st.n_resid = 0;
    }
    st.n_resid += 1;
    return st;
  }
  st.n_quant = st.n_resid = 0;
  bool same = true;
  for (int b = 0; b < c->cfg.batch; ++b) {
    if (st.sr[b] == R) {
      st.sq[b] += R;
      st.sr[b] = 0;
    }
    st.sr[b] += 1;
    st.n_quant = std::max(st.n_quant, st.sq[b]);
    st.n_resid = std::max(st.n_resid, st.sr[b]);
    same = same && st.sq[b] == st.sq[0] && st.sr[b] == st.sr[0];
  }
  if (same) {  // as settle(): equal lengths go back to the uniform state
    st.ragged = false;
    st.sq.clear();
    st.sr.clear();
  }
  return st;
}

// The compute-unit count of the current device (queried at creation, or
// here when that failed).  Nothing is enqueued; a failure leaves the cache
// unchanged.
kivi_status ensure_cu_count(kivi_cache* c) {
  if (c->cu_count > 0) return KIVI_OK;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus < 1)
    return fail(KIVI_ERR_HIP, "querying the compute-unit count: %s",
                e != hipSuccess ? hipGetErrorString(e) : "no compute units");
  c->cu_count = cus;
  return KIVI_OK;
}

// How a decode launch splits the token axis.
struct DecodePlan {
  int n_split, n_split_packed, gps, hg;
};

// Plans the decode launches over state `st` for gq query heads per kv head
// (pure host arithmetic: no device access, no change of the cache).
kivi_status plan_decode_uncached(const kivi_cache* c, const DecodeState& st, int gq, DecodePlan& out);

// plan_decode_uncached, reused while its inputs are unchanged: the state's
// longest packed length, whether a window exists, the packed length of each
// sequence (ragged), the head ratio, a forced split count and the
// compute-unit count.  The configuration is fixed per cache.
kivi_status plan_decode(const kivi_cache* c, const DecodeState& st, int gq, DecodePlan& out) {
  const int key[6] = {st.ragged ? 1 : 0, st.n_quant, st.n_resid > 0 ? 1 : 0, gq, c->forced_splits, c->cu_count};
  if (c->memo_valid && std::equal(key, key + 6, c->memo_key) && (!st.ragged || st.sq == c->memo_sq)) {
    out = DecodePlan{c->memo_plan[0], c->memo_plan[1], c->memo_plan[2], c->memo_plan[3]};
    return KIVI_OK;
  }
  const kivi_status r = plan_decode_uncached(c, st, gq, out);
  c->memo_valid = r == KIVI_OK;
  if (r == KIVI_OK) {
    std::copy(key, key + 6, c->memo_key);
    c->memo_sq = st.ragged ? st.sq : std::vector<int>();
    const int plan[4] = {out.n_split, out.n_split_packed, out.gps, out.hg};
    std::copy(plan, plan + 4, c->memo_plan);
  }
  return r;
}

kivi_status plan_decode_uncached(const kivi_cache* c, const DecodeState& st, int gq, DecodePlan& out) {
  // the kernel walks the packed tokens in streams of 32 (a block of G = 32,
  // or half a block of G = 64)
  const int G = kivi::kStream;
  const int units = c->cfg.batch * c->cfg.num_kv_heads;
  const int nqg = st.n_quant / G;
  // a workgroup serves up to 8 query heads of its kv head; 16 take 2
  // workgroups (head groups) per split
  const int hg = gq > 8 ? gq / 8 : 1;
  int n_split_packed = 0, gps = 0;
  // one workgroup (key wave + value wave) per split and head group; one
  // round of as many as fit in LDS on every CU, each split a multiple of 4
  // groups; the window is one more partial, computed by the workgroup of
  // the last packed split
  if (nqg > 0) {
    // resident workgroups per CU: LDS, and at most 6 (3 waves per SIMD at
    // the kernel's register budget)
    const int wgs_per_cu = std::max(
        1, std::min(6, kivi::kLdsPerCu / kivi::mfma_wg_lds_bytes(c->cfg.k_bits, c->cfg.v_bits, gq >= 8 ? 8 : 4)));
    const long long slots = (long long)wgs_per_cu * c->cu_count;
    const int max_split = std::max(1, std::min((nqg + 3) / 4, kivi::kMaxSplits - 1));
    auto plan = [&](int want, int& g, int& np) {
      g = ((nqg + want - 1) / want + 3) / 4 * 4;  // groups per split, whole steps of 4
      np = (nqg + g - 1) / g;
    };
    if (c->forced_splits > 0) {
      plan(std::min(c->forced_splits, max_split), gps, n_split_packed);
    } else {
      // minimise (rounds of resident workgroups) x (steps per workgroup):
      // every split of one launch takes the same time, so a partly filled
      // last round costs a whole workgroup duration
      // (sequences of different lengths: only the splits that hold groups
      // of their sequence count; the others end at once)
      // For ragged caches every multiple of 4 is a candidate split size
      // (the divisions of the longest sequence alone are too coarse to
      // fill a round with the shorter ones).
      long long best = -1;
      const int n_cand = st.ragged ? (nqg + 3) / 4 : max_split;
      // Ragged caches: the plans whose whole grid (the splits past a short
      // sequence's end included) fits in one round of resident slots are
      // preferred (a second round, even of short or empty splits, was
      // measured slower), and among them the one with the
      // smallest estimated time (steps per split + set-up) x (time of one
      // step).  A step takes the time of a lone workgroup or, with k
      // workgroups sharing a CU, k times the per-workgroup share of a fully
      // occupied CU, whichever is longer: the split kernel is bound by the
      // vector and matrix issue of its SIMDs.  In units of that share, a
      // lone workgroup's step is kLone x (workgroups per CU at full
      // occupancy): about 2.35 us against 3.7-4.1 us for a step of a full
      // CU on c2-shaped data.  Interleaved runs on ragged batches: c3 135-139
      // -> 115-125 us and c1 36.3-36.8 -> 33.0-33.9 us against the rounds
      // model above; c2 unchanged within noise.
      constexpr double kSetup = 1.5, kLone = 0.57;
      const double lone = kLone * wgs_per_cu;
      double best1 = -1.0;
      for (int i = 1; i <= n_cand; ++i) {
        int g, np;
        if (st.ragged) {
          g = 4 * i;
          np = (nqg + g - 1) / g;
          if (np > kivi::kMaxSplits - 1) continue;
        } else {
          plan(i, g, np);
        }
        long long work = (long long)units * np * hg;
        if (st.ragged) {
          work = 0;
          for (int b = 0; b < c->cfg.batch; ++b) work += (st.sq[b] / G + g - 1) / g;
          work *= (long long)c->cfg.num_kv_heads * hg;
          // (a ragged launch covers at most kDecodeChunk sequences)
          const long long grid =
              (long long)np * std::min(c->cfg.batch, kivi::kDecodeChunk) * c->cfg.num_kv_heads * hg;
          if (grid <= slots) {
            const double cost1 = (g / 4 + kSetup) * std::max(lone, work / (double)c->cu_count);
            if (best1 < 0.0 || cost1 < best1) {
              best1 = cost1;
              gps = g;
              n_split_packed = np;
            }
            continue;
          }
          if (best1 >= 0.0) continue;  // a one-round plan exists
        }
        const long long rounds = (work + slots - 1) / slots;
        const long long cost = rounds * (g / 4 + 1);  // +1: per-workgroup set-up and partial
        if (best1 < 0.0 && (best < 0 || cost < best)) {
          best = cost;
          gps = g;
          n_split_packed = np;
        }
      }
    }
  }
  const int n_split = n_split_packed + (st.n_resid > 0 ? 1 : 0);

  // the workspace query sized the partials for at most this many splits
  if (n_split > std::min(kivi::kMaxSplits, max_items(c)))
    return fail(KIVI_ERR_UNSUPPORTED, "internal: %d planned splits exceed the workspace bound %d", n_split,
                std::min(kivi::kMaxSplits, max_items(c)));
  out = DecodePlan{n_split, n_split_packed, gps, hg};
  return KIVI_OK;
}

// Launches decode attention over the cache's current state with a plan made
// for that state.  With k_new each unit's newest window token is read from
// k_new / v_new and stored into the window by the same launch.
kivi_status decode_launch(kivi_cache* c, const DecodePlan& plan, const void* q, int32_t num_q_heads,
                          float softmax_scale, void* out, int32_t out_dtype, void* workspace, void* stream,
                          const void* k_new, const void* v_new) {
  kivi::DecodeArgs a{};
  a.blocks = c->blocks;
  a.scale_max = c->scale_max;
  a.k_resid = c->k_resid;
  a.v_resid = c->v_resid;
  a.q = static_cast<const uint16_t*>(q);
  a.out = out;
  a.partial = static_cast<float*>(workspace);
  a.B = c->cfg.batch;
  a.H = c->cfg.num_kv_heads;
  a.Hq = num_q_heads;
  a.gq = num_q_heads / c->cfg.num_kv_heads;
  a.cap = c->cap;
  a.nb = c->nb;
  a.G = c->cfg.group_size;
  a.R = c->cfg.residual_length;
  a.n_quant = c->n_quant;
  a.n_resid = c->n_resid;
  a.n_split = plan.n_split;
  a.n_split_packed = plan.n_split_packed;
  a.groups_per_split = plan.gps;
  a.hg = plan.hg;
  a.qscale = softmax_scale * 1.4426950408889634f;  // log2(e): base-2 softmax
  a.page_table = c->page_table;
  a.page_stride = c->page_stride;
  a.num_pages = c->num_pages;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_resid_w = c->k_resid;
  a.v_resid_w = c->v_resid;
  if (!c->ragged) {
    hipError_t e = kivi::launch_decode(a, c->cfg.k_bits, c->cfg.v_bits, c->cfg.kv_dtype, out_dtype,
                                       static_cast<hipStream_t>(stream), c->ev_split_begin,
                                       c->ev_split_end);
    if (e != hipSuccess) return hip_fail(c, e, "decode launch");
    return KIVI_OK;
  }
  // sequences of different lengths: the splits are planned for the longest
  // (n_quant, n_resid hold the largest); each launch covers kDecodeChunk
  // sequences with their own lengths, and splits past a sequence's end
  // leave empty partials
  a.ragged = 1;
  for (int b0 = 0; b0 < c->cfg.batch; b0 += kivi::kDecodeChunk) {
    const int nseq = std::min(kivi::kDecodeChunk, c->cfg.batch - b0);
    a.seq0 = b0;
    a.B = nseq;
    for (int i = 0; i < nseq; ++i) {
      a.seq_len[i][0] = c->sq[b0 + i];
      a.seq_len[i][1] = c->sr[b0 + i];
    }
    hipError_t e = kivi::launch_decode(a, c->cfg.k_bits, c->cfg.v_bits, c->cfg.kv_dtype, out_dtype,
                                       static_cast<hipStream_t>(stream), c->ev_split_begin,
                                       c->ev_split_end);
    if (e != hipSuccess) return hip_fail(c, e, "decode launch (sequences of different lengths)");
  }
  return KIVI_OK;
}

}  // namespace

extern "C" {

kivi_status kivi_decode_attn(kivi_cache* c, const void* q, int32_t num_q_heads, float softmax_scale,
                             void* out, int32_t out_dtype, void* workspace, size_t ws_bytes,
                             void* stream) {
  kivi_status st = check_decode_args(c, q, num_q_heads, out, out_dtype, workspace, ws_bytes);
  if (st != KIVI_OK) return st;
  if (c->n_quant + c->n_resid < 1) return fail(KIVI_ERR_EMPTY, "decode on an empty cache");
  if ((st = ensure_cu_count(c)) != KIVI_OK) return st;
  DecodePlan plan;
  if ((st = plan_decode(c, state_of(c), num_q_heads / c->cfg.num_kv_heads, plan)) != KIVI_OK) return st;
  return decode_launch(c, plan, q, num_q_heads, softmax_scale, out, out_dtype, workspace, stream, nullptr,
                       nullptr);
}

}  // extern "C"

kivi_status kivi::report(kivi_status s, const char* message) { return fail(s, "%s", message); }

kivi_status kivi::decode_attn_bounded(kivi_cache* c, const void* q, int32_t num_q_heads, float softmax_scale,
                                      void* out, int32_t out_dtype, void* scratch, size_t scratch_bytes,
                                      void* stream) {
  // the checks of kivi_decode_attn, with the workspace bound by the plan
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (c->poisoned) return fail(KIVI_ERR_HIP, "cache handle is poisoned by an earlier HIP error");
  if (!q || !out) return fail(KIVI_ERR_INVALID_ARG, "q and out must not be NULL");
  if (num_q_heads < 1 || num_q_heads % c->cfg.num_kv_heads)
    return fail(KIVI_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, c->cfg.num_kv_heads);
  if (out_dtype != KIVI_F16 && out_dtype != KIVI_BF16 && out_dtype != KIVI_F32)
    return fail(KIVI_ERR_INVALID_ARG, "bad out_dtype %d", out_dtype);
  const int gq = num_q_heads / c->cfg.num_kv_heads;
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8 && gq != 16)
    return fail(KIVI_ERR_UNSUPPORTED, "query heads per kv head must be 1, 2, 4, 8 or 16 (got %d)", gq);
  if (c->n_quant + c->n_resid < 1) return fail(KIVI_ERR_EMPTY, "decode on an empty cache");
  kivi_status st;
  if ((st = ensure_cu_count(c)) != KIVI_OK) return st;
  DecodePlan plan;
  if ((st = plan_decode(c, state_of(c), gq, plan)) != KIVI_OK) return st;
  const size_t need = workspace_bytes_for(c, num_q_heads, plan.n_split);
  if (need > scratch_bytes)
    return fail(KIVI_ERR_BUFFER_TOO_SMALL,
                "the planned partials need %zu bytes, more than the %zu of the fixed scratch array", need,
                scratch_bytes);
  return decode_launch(c, plan, q, num_q_heads, softmax_scale, out, out_dtype, scratch, stream, nullptr,
                       nullptr);
}

extern "C" {

kivi_status kivi_append_decode_attn(kivi_cache* c, const void* k_new, const void* v_new,
                                    const void* q, int32_t num_q_heads, float softmax_scale,
                                    void* out, int32_t out_dtype, void* workspace, size_t ws_bytes,
                                    void* stream) {
  kivi_status st = check_decode_args(c, q, num_q_heads, out, out_dtype, workspace, ws_bytes);
  if (st != KIVI_OK) return st;
  if (!k_new || !v_new) return fail(KIVI_ERR_INVALID_ARG, "k_new and v_new must not be NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(KIVI_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  int longest = c->n_quant + c->n_resid;
  if (c->ragged) {
    longest = 0;
    for (int b = 0; b < c->cfg.batch; ++b) longest = std::max(longest, c->sq[b] + c->sr[b]);
  }
  if ((long long)longest + 1 > c->cfg.max_tokens)
    return fail(KIVI_ERR_CAPACITY, "appending a token to %d exceeds max_tokens %d", longest,
                c->cfg.max_tokens);
  // everything that can fail without a launch failing is settled before the
  // first launch: the device query and the split plan of the state after the
  // token append
  if ((st = ensure_cu_count(c)) != KIVI_OK) return st;
  const int gq = num_q_heads / c->cfg.num_kv_heads;
  DecodePlan plan;
  if ((st = plan_decode(c, after_token(c), gq, plan)) != KIVI_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = c->cfg.residual_length;
  // A full window is packed before the token enters it (a launch of its
  // own, once every R steps); then the token takes the next window slot.
  // (Packing it inside the decode launch, by the workgroup of the last split,
  // was measured slower at every workload: that workgroup's 4 blocks in a
  // row outlast the separate launch.)
  if (c->ragged) {
    std::vector<char> fl(c->cfg.batch, 0);
    for (int b = 0; b < c->cfg.batch; ++b) fl[b] = c->sr[b] == R;
    if ((st = ragged_flush(c, fl, s)) != KIVI_OK) return st;
    for (int b = 0; b < c->cfg.batch; ++b) c->sr[b] += 1;
    settle(c);
  } else {
    if (c->n_resid == R && (st = flush_window(c, s)) != KIVI_OK) return st;
    c->n_resid += 1;
  }
  return decode_launch(c, plan, q, num_q_heads, softmax_scale, out, out_dtype, workspace, stream, k_new,
                       v_new);
}

kivi_status kivi_cache_set_lengths(kivi_cache* c, const int32_t* n_quant, const int32_t* n_resid) {
  if (!c || !n_quant || !n_resid) return fail(KIVI_ERR_INVALID_ARG, "cache and lengths must not be NULL");
  if (c->poisoned) return fail(KIVI_ERR_HIP, "cache handle is poisoned by an earlier HIP error");
  const int B = c->cfg.batch, R = c->cfg.residual_length;
  for (int b = 0; b < B; ++b) {
    if (n_quant[b] < 0 || n_quant[b] % R != 0 || n_resid[b] < 0 || n_resid[b] > R ||
        (long long)n_quant[b] + n_resid[b] > c->cfg.max_tokens)
      return fail(KIVI_ERR_INVALID_ARG,
                  "sequence %d: lengths (%d, %d) need n_quant a multiple of R = %d, 0 <= n_resid <= R and "
                  "n_quant + n_resid <= max_tokens = %d", b, n_quant[b], n_resid[b], R, c->cfg.max_tokens);
  }
  c->ragged = true;
  c->sq.assign(n_quant, n_quant + B);
  c->sr.assign(n_resid, n_resid + B);
  settle(c);
  return KIVI_OK;
}

kivi_status kivi_set_timing_events(kivi_cache* c, void* split_begin, void* split_end) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if ((split_begin == nullptr) != (split_end == nullptr))
    return fail(KIVI_ERR_INVALID_ARG, "give both events or neither");
  c->ev_split_begin = static_cast<hipEvent_t>(split_begin);
  c->ev_split_end = static_cast<hipEvent_t>(split_end);
  return KIVI_OK;
}

kivi_status kivi_stream_read_probe(const void* src, size_t bytes, void* sink, size_t sink_bytes,
                                   int32_t workgroups, void* stream) {
  if (!src || !sink) return fail(KIVI_ERR_INVALID_ARG, "src and sink must not be NULL");
  if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return fail(KIVI_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 and src 16-byte aligned");
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(KIVI_ERR_INVALID_ARG, "workgroups must be in [1, 2^20]");
  if (sink_bytes < (size_t)workgroups * 256 * 4)
    return fail(KIVI_ERR_BUFFER_TOO_SMALL, "sink needs %zu bytes", (size_t)workgroups * 256 * 4);
  hipError_t e = kivi::launch_stream_read(src, bytes, static_cast<uint32_t*>(sink), workgroups,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KIVI_ERR_HIP, "stream read launch: %s", hipGetErrorString(e));
  return KIVI_OK;
}

kivi_status kivi_set_decode_splits(kivi_cache* c, int32_t n_split) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "cache is NULL");
  if (n_split < 0) return fail(KIVI_ERR_INVALID_ARG, "n_split must be >= 0");
  c->forced_splits = n_split;
  return KIVI_OK;
}

kivi_status kivi_cache_get_view(const kivi_cache* c, kivi_cache_view* v) {
  if (!c || !v) return fail(KIVI_ERR_INVALID_ARG, "cache and view must not be NULL");
  v->n_quant = c->ragged ? -1 : c->n_quant;  // per sequence: kivi_cache_get_lengths
  v->n_resid = c->ragged ? -1 : c->n_resid;
  v->capacity = c->cap;
  v->num_blocks = c->nb;
  const kivi::BlockLayout bl = kivi::block_layout(c->cfg.k_bits, c->cfg.v_bits, c->cfg.group_size);
  v->block_bytes = bl.bytes;
  v->off_k_codes = bl.k_codes;
  v->off_v_codes = bl.v_codes;
  v->off_k_scale = bl.k_scale;
  v->off_k_zero = bl.k_zero;
  v->off_v_scale = bl.v_scale;
  v->off_v_zero = bl.v_zero;
  v->blocks = c->blocks;
  v->k_resid = c->k_resid;
  v->v_resid = c->v_resid;
  v->scale_max = c->scale_max;
  return KIVI_OK;
}

const char* kivi_status_string(kivi_status s) {
  switch (s) {
    case KIVI_OK: return "KIVI_OK";
    case KIVI_ERR_INVALID_ARG: return "KIVI_ERR_INVALID_ARG";
    case KIVI_ERR_UNSUPPORTED: return "KIVI_ERR_UNSUPPORTED";
    case KIVI_ERR_CAPACITY: return "KIVI_ERR_CAPACITY";
    case KIVI_ERR_BUFFER_TOO_SMALL: return "KIVI_ERR_BUFFER_TOO_SMALL";
    case KIVI_ERR_EMPTY: return "KIVI_ERR_EMPTY";
    case KIVI_ERR_HIP: return "KIVI_ERR_HIP";
  }
  return "unknown kivi_status";
}

const char* kivi_last_error_message(void) { return g_last_error.c_str(); }

}  // extern "C"
