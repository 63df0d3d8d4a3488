/*
 * kivi.h - C ABI of the KIVI hot path on AMD Instinct MI355X (gfx950).
 *
 * KIVI keeps the attention KV cache of a decoder in low-bit integer codes:
 *   - keys are quantized per channel: the G consecutive tokens of one channel
 *     form a group with its own scale and zero-point
 *     (page "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide", section
 *     "The Three Structural Innovations of KIVI", item 1; page "KV cache
 *     quantization with KIVI INT2 setup guide", section "KIVI: Per-Channel Key,
 *     Per-Token Value Quantization Explained", defaults G=32, R=128);
 *   - values are quantized per token: the G consecutive channels of one token
 *     form a group (same pages, item 2 / same section);
 *   - the newest R tokens stay unquantized in a residual window; when the
 *     window is full it is quantized and packed as a whole ("Asymmetric 2-Bit"
 *     guide, item 3 "The Streaming Residual FP16 Window");
 *   - decode attention reads the packed codes and dequantizes them on the fly
 *     ("Asymmetric 2-Bit" guide, section "Production Serving and vLLM
 *     Deployment Trade-offs"; page "KV-Cache Quantization: I Ran the
 *     Experiments", section "Where it still breaks", item 3).
 *
 * Quantizer of one group x_0..x_{G-1} (b bits, qmax = 2^b - 1), in binary32
 * with round-to-nearest-even on every operation ("Asymmetric 2-Bit" guide,
 * "Step 1" and "Step 2"; zero-point kept as a float, see the design notes):
 *     mn = min x_j,  mx = max x_j,  s = (mx - mn) / qmax
 *     c_j = clamp(rne((x_j - mn) / s), 0, qmax)      (all c_j = 0 when s == 0)
 *     S = fp16(s), Z = fp16(mn)   (a zero S or Z is stored as +0, bits 0x0000)
 *     dequantized value  x^_j = c_j * S + Z
 *
 * ------------------------------------------------------------------------
 * Packed layout (all arrays are per cache = one attention layer).
 *   B = batch, H = KV heads, D = head_dim, G = group_size, R = residual_length,
 *   cap = max_tokens rounded up to a multiple of R, NB = cap / G blocks,
 *   bk = k_bits, bv = v_bits, Pk = 32 / bk and Pv = 32 / bv codes per word.
 * A "unit" is one (batch b, kv head h) pair, unit index u = b * H + h.
 * Token t of a unit lies in block g = t / G at row j = t % G.
 *
 * Word bit order ("split-half"): code number i (0 <= i < P) of a 32-bit word
 * occupies bits [o, o + bits) with o = bits * (i / 2) + 16 * (i % 2): even
 * codes fill the low half-word, odd codes the high half-word, each half in
 * increasing order.  Masking a word with 0x00030003 (2-bit) or 0x000F000F
 * (4-bit) after a shift therefore yields two codes, one per 16-bit lane.
 *
 * Codes are packed along the axis that the attention contraction runs over
 * (channels for q.K, tokens for p.V), not along the quantization group.
 *
 * Every (unit u, block g) of packed tokens is one contiguous record of
 *   block_bytes = G*D*bk/8 + G*D*bv/8 + 8*D
 * bytes at  blocks + (u * NB + g) * block_bytes  (3 KiB for D = 128, G = 32,
 * 2-bit keys and values), so that a decode step streams one region:
 *   offset                        field    type / shape
 *   0                             k_codes  uint32 [G][D / Pk]   word w of row
 *                                          j holds channels w*Pk .. w*Pk+Pk-1
 *   G*D*bk/8                      v_codes  uint32 [G / Pv][D]   word (w, d)
 *                                          holds rows w*Pv .. w*Pv + Pv - 1 of
 *                                          channel d; the D words of one w are
 *                                          adjacent
 *   + G*D*bv/8                    k_scale  fp16 [D]     {S} per channel
 *   + 2*D                         k_zero   fp16 [D]     {Z} per channel
 *                                          (both interleaved: position i of
 *                                          the 8 channels 8j .. 8j+7 holds
 *                                          channel 8j + i/2 + 4 (i mod 2),
 *                                          so word w holds channels 8j + w
 *                                          and 8j + w + 4)
 *   + 4*D                         v_scale  fp16 [D / G][G]  {S} per (channel
 *                                          group, row)
 *   + 6*D                         v_zero   fp16 [D / G][G]
 * The residual window is stored apart:
 *   k_resid, v_resid  kv_dtype [B*H][R][D]  slot i holds the token
 *                                          n_quant + i
 * and so is one 32-bit word per block record, at the record's index:
 *   scale_max  uint32 [B*H*NB]  bits 0-15: the largest k_scale of the
 *                               record, bits 16-31: the largest v_scale
 *                               (fp16 bit patterns; scales are >= 0)
 * The decode reads these maxima to keep its fp16 matrix operands in range.
 * Tokens [0, n_quant) are packed, tokens [n_quant, n_quant + n_resid) are in
 * the residual window.  Entries beyond those are unspecified.
 *
 * ------------------------------------------------------------------------
 * Conventions for every entry point.
 *   - All device memory is owned by the caller (cache buffer, inputs, q, out,
 *     workspace) and must stay alive until the stream work that uses it has
 *     finished.  The library never allocates or frees device memory and never
 *     creates streams; it owns only the host-side kivi_cache struct.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Calls enqueue work and return without synchronizing.  Host-side counters
 *     (n_quant, n_resid) advance at enqueue time, so all calls on one cache
 *     must be issued in order on one stream.  A cache handle is not
 *     thread-safe.
 *   - Argument errors are detected before anything is enqueued; the call then
 *     returns the error and leaves the cache unchanged.  A failed kernel
 *     launch returns KIVI_ERR_HIP and poisons the handle (later calls return
 *     KIVI_ERR_HIP).  Device faults surface at the caller's next
 *     synchronization.  kivi_last_error_message() gives a thread-local text.
 *   - Inputs (k, v and q) must be finite and within +-65504, the fp16 range
 *     of the stored scale S and zero-point Z; results for other inputs are
 *     unspecified.
 */
#ifndef KIVI_H_
#define KIVI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kivi_cache kivi_cache; /* opaque host handle, one per layer */

typedef enum {
  KIVI_OK = 0,
  KIVI_ERR_INVALID_ARG = 1,      /* null pointer, malformed config or size */
  KIVI_ERR_UNSUPPORTED = 2,      /* valid, but not built (e.g. head_dim != 128) */
  KIVI_ERR_CAPACITY = 3,         /* more tokens than max_tokens */
  KIVI_ERR_BUFFER_TOO_SMALL = 4, /* cache buffer or workspace too small */
  KIVI_ERR_EMPTY = 5,            /* decode on a cache that holds no token */
  KIVI_ERR_HIP = 6               /* a HIP call failed; handle is poisoned */
} kivi_status;

typedef enum { KIVI_F16 = 0, KIVI_BF16 = 1, KIVI_F32 = 2 } kivi_dtype;

/* Quantization config: the knobs k_bits, v_bits, group_size and
 * residual_length of page "KV-Cache Quantization: I Ran the Experiments",
 * section "Component 4 - Serving architecture & manifests". */
typedef struct {
  int32_t batch;           /* B >= 1 */
  int32_t num_kv_heads;    /* H >= 1 */
  int32_t head_dim;        /* D; multiple of group_size. Kernels: 128 */
  int32_t max_tokens;      /* per-sequence capacity T_max >= 1 */
  int32_t k_bits;          /* 2 or 4 */
  int32_t v_bits;          /* 2 or 4 */
  int32_t group_size;      /* G. Kernels: 32 or 64 */
  int32_t residual_length; /* R; positive multiple of G, at most 1024 */
  int32_t kv_dtype;        /* kivi_dtype: KIVI_F16 or KIVI_BF16 (inputs,
                              residual window and q) */
} kivi_config;

/* Device pointers into the cache buffer plus the host counters. */
typedef struct {
  int32_t n_quant;     /* tokens packed; a multiple of R (-1 while the
                          sequences hold different lengths: see
                          kivi_cache_get_lengths) */
  int32_t n_resid;     /* tokens in the residual window, 0..R (-1 likewise) */
  int32_t capacity;    /* cap: max_tokens rounded up to a multiple of R */
  int32_t num_blocks;  /* NB = cap / G */
  int32_t block_bytes; /* bytes of one block record */
  /* byte offsets of the fields inside a block record */
  int32_t off_k_codes, off_v_codes, off_k_scale, off_k_zero, off_v_scale, off_v_zero;
  void* blocks;        /* [B*H][NB] block records */
  void *k_resid, *v_resid; /* kv_dtype */
  void* scale_max;     /* uint32 [B*H*NB]: per record, largest key scale
                          (low half) and value scale (high half) */
} kivi_cache_view;

/* Bytes of device memory the cache for `cfg` needs (the block records, the
 * two window arrays and the per-record scale maxima, each 256-byte aligned).
 * Pure arithmetic; no device is touched. */
kivi_status kivi_cache_bytes(const kivi_config* cfg, size_t* bytes);

/* Creates an empty cache (n_quant = n_resid = 0) for one attention layer
 * over the caller's device buffer `dev_buf` of `dev_bytes` bytes
 * (>= kivi_cache_bytes, 256-byte aligned): the per-layer store of packed
 * keys and values plus the full-precision window that the cache manager of
 * page "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide", "Step 3:
 * Implement the KIVI KV Cache Manager with Rolling Window", keeps.  The
 * buffer content is not read or written here; the current device's
 * compute-unit count is queried (a failed query is repeated by the first
 * decode).  On success *out receives a handle the caller frees with
 * kivi_cache_destroy.
 * Errors: those of kivi_cache_bytes, INVALID_ARG (null dev_buf or out,
 * unaligned dev_buf), BUFFER_TOO_SMALL. */
kivi_status kivi_cache_create(const kivi_config* cfg, void* dev_buf,
                              size_t dev_bytes, kivi_cache** out);

/* Frees the host handle.  Does not synchronize and does not touch the
 * device buffer.  NULL is accepted. */
kivi_status kivi_cache_destroy(kivi_cache* cache);

/* Forgets every token (n_quant = n_resid = 0) without touching device
 * memory, so the buffer can be refilled. */
kivi_status kivi_cache_reset(kivi_cache* cache);

/* Appends n_tokens tokens per sequence.  k and v are device arrays of
 * kv_dtype laid out [B][H][n_tokens][D] (page "KIVI: Asymmetric 2-Bit KV Cache
 * Quantization Guide", "Step 1", tensor layout [batch, heads, seq_len,
 * head_dim]).  The result is, bit for bit, that of n_tokens single-token
 * appends, each of which first packs the residual window if it holds R
 * tokens and then stores the token in the window ("Step 3" and item 3 of
 * "The Three Structural Innovations of KIVI").  Afterwards
 * 1 <= n_resid <= R (for n_tokens >= 1) and n_quant % R == 0.
 * Full windows inside the input are packed straight from k/v.
 * Errors: INVALID_ARG (null cache/k/v, n_tokens < 0), CAPACITY (total would
 * exceed max_tokens), HIP.  n_tokens == 0 is a no-op. */
kivi_status kivi_append(kivi_cache* cache, const void* k, const void* v,
                        int32_t n_tokens, void* stream);

/* Appends n_tokens[b] tokens to sequence b (0 <= n_tokens[b] <= n_max, a
 * host array of `batch` entries).  k and v are device arrays of kv_dtype laid
 * out [B][H][n_max][D]; sequence b takes its first n_tokens[b] tokens.  Each
 * sequence follows the rules of kivi_append on its own lengths, so sequences
 * may hold different lengths afterwards (many concurrent requests, each with
 * its own cache: page "KV cache quantization with KIVI INT2 setup guide",
 * section "VRAM Before/After and What It Buys You in Batch Size").  The work
 * runs as at most four launches per 32 sequences.  kivi_append on such a
 * cache appends n_tokens to every sequence.
 * Errors: INVALID_ARG (null cache/n_tokens, n_tokens[b] outside [0, n_max],
 * null or unaligned k/v when some n_tokens[b] > 0), CAPACITY (a sequence
 * would exceed max_tokens; nothing is appended), HIP. */
kivi_status kivi_append_varlen(kivi_cache* cache, const void* k, const void* v,
                               const int32_t* n_tokens, int32_t n_max, void* stream);

/* Forgets every token of the `count` sequences listed in seqs (host array),
 * without touching device memory; their next append starts from an empty
 * cache (a finished request's slot taken by a new one).
 * Errors: INVALID_ARG (null cache, null seqs with count > 0, an index
 * outside [0, batch)). */
kivi_status kivi_cache_reset_sequences(kivi_cache* cache, const int32_t* seqs, int32_t count);

/* Paged block records.  With a table set, block g (tokens G g .. G g + G - 1)
 * of sequence b lives in page P = table[b * page_stride + g] of the block
 * region, and kv head h of it at record P * H + h (the region then holds
 * num_pages pages of H records; the default is the unit-major layout,
 * record (b * H + h) * NB + g).  A caller that manages its own page
 * allocation (quantized blocks in paged KV memory: page "KV-Cache
 * Quantization: I Ran the Experiments So You Don't Have To", "Component 4 -
 * Serving architecture & manifests", Figure 8) maps each sequence's blocks
 * to free pages and may hand a freed page to another sequence.
 * `table` is a device array of int32 [B][page_stride] that must stay valid
 * and unchanged while work using it is in flight; the kernels read it and
 * clamp every entry into [0, num_pages), so a wrong table gives wrong results
 * but never touches memory outside the region.  Entries are needed for the
 * blocks a sequence holds.  NULL restores the unit-major layout.  Changing
 * the layout of a cache that holds packed tokens reinterprets them.
 * Errors: INVALID_ARG (null cache, page_stride < NB, num_pages outside
 * [1, batch * NB], unaligned table). */
kivi_status kivi_cache_set_page_table(kivi_cache* cache, const int32_t* table,
                                      int32_t page_stride, int32_t num_pages);

/* Per-sequence counters: n_quant[b] and n_resid[b] for b < batch (host
 * arrays).  Equal to the view's counters while every sequence has the same
 * lengths. */
kivi_status kivi_cache_get_lengths(const kivi_cache* cache, int32_t* n_quant, int32_t* n_resid);

/* Packs the residual window of every sequence whose window holds exactly R
 * tokens (n_quant += R, n_resid = 0); the others are left alone.  This is
 * the step of page "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide",
 * item 3 of "The Three Structural Innovations of KIVI" (tokens that leave
 * the streaming window are grouped and packed) and "Step 3", done for the
 * whole window at once, with the quantizer of "Step 1".  kivi_append runs
 * it by itself before a token enters a full window; calling it early only
 * moves that launch.
 * Errors: INVALID_ARG (null cache), HIP. */
kivi_status kivi_flush_residual(kivi_cache* cache, void* stream);

/* Workspace bytes kivi_decode_attn needs for num_q_heads query heads at any
 * fill level of this cache: the per-split partial softmax states (m, l,
 * o[D]) in fp32 of the split-K decode that reads the whole cache for every
 * generated token (page "KV-Cache Quantization: I Ran the Experiments So
 * You Don't Have To", "Component 1 - The cache is a tax that scales with
 * tokens").  Pure arithmetic.
 * Errors: INVALID_ARG (null cache or bytes, num_q_heads not a positive
 * multiple of num_kv_heads). */
kivi_status kivi_decode_attn_workspace_bytes(const kivi_cache* cache,
                                             int32_t num_q_heads,
                                             size_t* bytes);

/* One decode step of attention for every sequence (page "KIVI: Asymmetric
 * 2-Bit KV Cache Quantization Guide", "Step 2: Implement Dequantization for
 * Attention Computation", with the dequantization fused into the attention
 * kernel as its "Production Serving and vLLM Deployment Trade-offs" section
 * and page "KV-Cache Quantization: I Ran the Experiments", "Where it still
 * breaks", item 3, require; the paper abstract, "KIVI: A Tuning-Free
 * Asymmetric 2bit Quantization for KV Cache", for the loading of the cache
 * as what bounds the speed):
 *   out[b][j] = sum_t softmax_t(softmax_scale * q[b][j] . k^_t) v^_t
 * over the T = n_quant + n_resid cached tokens of kv head h = j / (Hq / H)
 * (consecutive query heads share a kv head), where k^ and v^ are the
 * dequantized codes for packed tokens and the stored kv_dtype values for
 * window tokens.  q is a device array of kv_dtype [B][Hq][D]; out is a
 * device array of out_dtype (KIVI_F32, KIVI_F16 or KIVI_BF16) [B][Hq][D].
 * The token axis is split across workgroups and the per-split partial
 * softmax states are merged exactly (log-sum-exp) in a second kernel; the
 * workspace holds those partials.
 * The products run on the matrix cores with fp16 operands (hi + lo pairs,
 * about 22 significant bits); one workgroup serves up to 8 query heads of a
 * kv head per token split, so 16 query heads per kv head take 2 workgroups
 * over the same records.  Each workgroup scales its folded operands q*S and p*S by powers of two chosen
 * from the largest |q| of each head and the scale maxima of the records it
 * reads, so every input in the domain stated above stays in the operands'
 * range; the scaling is exact and undone in fp32.
 * Sequences of different lengths each attend over their own tokens; a
 * sequence without tokens gets zeros.  The splits are then planned for the
 * longest sequence, and each launch pair covers 64 sequences.
 * Errors: INVALID_ARG (nulls, Hq not a positive multiple of H, bad dtype),
 * UNSUPPORTED (a ratio Hq / H other than 1, 2, 4, 8 or 16),
 * EMPTY (no sequence holds a token), BUFFER_TOO_SMALL (ws_bytes below the
 * workspace query), HIP (the compute-unit query failed: nothing enqueued,
 * cache unchanged; or the launch failed: the handle is poisoned). */
kivi_status kivi_decode_attn(kivi_cache* cache, const void* q,
                             int32_t num_q_heads, float softmax_scale,
                             void* out, int32_t out_dtype, void* workspace,
                             size_t ws_bytes, void* stream);

/* One decode step: appends one token per sequence (k_new, v_new: device
 * arrays of kv_dtype [B][H][D]) exactly as kivi_append with n_tokens = 1,
 * then runs kivi_decode_attn over the cache including that token (the
 * residual-window append and decode attention of one generated token, page
 * "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide", "Step 3").  The
 * token is read from k_new / v_new and stored into the window by the
 * attention launch itself: one launch fewer than the two calls.  A full
 * window is still packed first, in a launch of its own.
 * Errors: those of kivi_decode_attn and kivi_append (INVALID_ARG for null or
 * unaligned k_new / v_new, CAPACITY).  The argument checks, the device query
 * and the split plan of the state after the append all come before anything
 * is enqueued or counted, so these errors leave the cache unchanged; a failed
 * launch poisons the handle. */
kivi_status kivi_append_decode_attn(kivi_cache* cache, const void* k_new, const void* v_new,
                                    const void* q, int32_t num_q_heads, float softmax_scale,
                                    void* out, int32_t out_dtype, void* workspace,
                                    size_t ws_bytes, void* stream);

/* Declares that the cache buffer holds, for every sequence b, n_quant[b]
 * packed tokens and n_resid[b] window tokens (host arrays of `batch`
 * entries), without touching device memory: a buffer restored from a
 * snapshot of this cache (its bytes copied back, or saved and reloaded)
 * resumes at the lengths it had, the same state kivi_cache_get_lengths
 * reported when the snapshot was taken.  The contents are not checked.
 * Errors: INVALID_ARG (nulls; n_quant[b] not a non-negative multiple of R,
 * n_resid[b] outside [0, R], or n_quant[b] + n_resid[b] > max_tokens), HIP
 * (poisoned handle). */
kivi_status kivi_cache_set_lengths(kivi_cache* cache, const int32_t* n_quant,
                                   const int32_t* n_resid);

/* kivi_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  The split partials go to a fixed 16 MiB
 * device array inside the library (one per GPU, held until the process
 * ends; its address is looked up once per device, on the first call with
 * that device current); the call allocates nothing.  Same kernels, plan and
 * results as kivi_decode_attn.  Calls on one GPU share the array, so calls
 * that overlap on one GPU (other streams, other threads) race; issue them in
 * order on one stream.
 * Errors: those of kivi_decode_attn except the workspace ones;
 * BUFFER_TOO_SMALL when the planned partials (batch * num_q_heads * splits *
 * (head_dim + 2) * 4 bytes) exceed the array, before anything is enqueued. */
kivi_status kivi_decode_attn_noalloc(kivi_cache* cache, const void* q, int32_t num_q_heads,
                                     float softmax_scale, void* out, int32_t out_dtype, void* stream);

/* Fixes the number of token splits used by kivi_decode_attn (0 restores the
 * automatic choice).  The value is clamped to [1, blocks + 1]. For tests of
 * split invariance and for tuning. */
kivi_status kivi_set_decode_splits(kivi_cache* cache, int32_t n_split);

/* Fills *view with the device pointers and counters of the cache. */
kivi_status kivi_cache_get_view(const kivi_cache* cache, kivi_cache_view* view);

/* ------------------------------------------------------------------------
 * Measurement helpers (for benchmarks and profiling; not part of the path).
 */

/* Timing hook: with events set, every decode launch on this cache records
 * split_begin on its stream right before the split-K attention kernel and
 * split_end right after it, before the merge (hipEvent_t handles passed as
 * void*, created by the caller; both or neither; NULL, NULL removes them).
 * Each record is a stream marker, so a marked launch starts a little later
 * than an unmarked one; events created with hipEventDisableSystemFence skip
 * the cache write-back and invalidation a default event's record performs,
 * and bracket the kernel more tightly.  For caches of more than 64 sequences of different
 * lengths the events bracket the last launch pair's split kernel.
 * Errors: INVALID_ARG (null cache, only one event given). */
kivi_status kivi_set_timing_events(kivi_cache* cache, void* split_begin, void* split_end);

/* Streaming-read probe: reads `bytes` (a positive multiple of 16) of device
 * memory at src (16-byte aligned) once with 16-byte non-temporal loads, by
 * `workgroups` workgroups of 256 threads each reading one contiguous chunk,
 * and writes one word per thread to the device array sink (at least
 * workgroups * 1024 bytes).  Timed by the caller, it gives the HBM read rate
 * a plain streaming kernel reaches: the practical ceiling for the decode,
 * which streams the packed cache once per generated token (page "KV-Cache
 * Quantization: I Ran the Experiments So You Don't Have To", "Component 1").
 * Errors: INVALID_ARG, BUFFER_TOO_SMALL (sink), HIP (launch failure). */
kivi_status kivi_stream_read_probe(const void* src, size_t bytes, void* sink, size_t sink_bytes,
                                   int32_t workgroups, void* stream);

/* Static text for a status code. */
const char* kivi_status_string(kivi_status status);

/* Thread-local detail for the last non-OK status returned on this thread. */
const char* kivi_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H_ */
