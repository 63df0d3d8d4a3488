/*
 * kivi_oracle.h - plain, slow CPU oracle of the KIVI hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package
 * entry file and the CPU-baseline leg of the benchmark may load or call this
 * library.  The product path (the HIP library and its Python binding) never
 * touches it, and it shares no code with that path.
 *
 * Every floating-point step of the quantizer is one binary32 operation with
 * round-to-nearest-even (the file is built with -ffp-contract=off and without
 * fast-math); attention is evaluated in binary64.
 *
 * Sources (web pages on KIVI, cited by title and section):
 *   [G]  "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide"
 *   [S]  "KV cache quantization with KIVI INT2 setup guide"
 *   [E]  "KV-Cache Quantization: I Ran the Experiments So You Don't Have To"
 *   [A]  "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 *        (paper abstract)
 *
 * Parity status: every function here is pinned by CPU tests against hand
 * derivations, closed forms, an exact-rational reference and textbook special
 * cases, except the attention values on synthetic data beyond those special
 * cases, for which no page prints numbers.
 */
#ifndef KIVI_ORACLE_H_
#define KIVI_ORACLE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact binary16 -> binary32, bfloat16 -> binary32 and round-to-nearest-even
 * binary32 -> binary16 conversions. */
float oracle_f16_to_f32(uint16_t h);
float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float f);

/* One quantization group ([G] "Step 1", asymmetric min/max quantizer; zero
 * point kept as the group minimum so that a constant group is exact).
 * x: n binary32 values.  Writes n codes, S and Z (binary16 bit patterns). */
void oracle_quantize_group(const float* x, int n, int bits, uint8_t* codes,
                           uint16_t* scale_f16, uint16_t* zero_f16);

/* Dequantized value c * S + Z in binary64 (exact). [G] "Step 2". */
double oracle_dequant(int code, uint16_t scale_f16, uint16_t zero_f16);

typedef struct {
  /* config */
  int B, H, D, T_max, kb, vb, G, R, dtype; /* dtype: 0 fp16, 1 bf16 */
  /* derived */
  int cap, nb;
  /* state */
  int n_quant, n_resid;
  /* host arrays in the packed layout (one unit = one (batch, kv head)) */
  uint32_t* k_codes; /* [B*H][cap][D*kb/32] */
  uint16_t* k_scale; /* [B*H][nb][D] */
  uint16_t* k_zero;  /* [B*H][nb][D] */
  uint32_t* v_codes; /* [B*H][nb][G*vb/32][D] */
  uint16_t* v_scale; /* [B*H][nb][D/G][G] */
  uint16_t* v_zero;  /* [B*H][nb][D/G][G] */
  uint16_t* k_resid; /* [B*H][R][D] */
  uint16_t* v_resid; /* [B*H][R][D] */
} oracle_cache;

/* Returns 0 on success, -1 on a bad config or allocation failure. */
int oracle_cache_init(oracle_cache* c, int B, int H, int D, int T_max, int kb,
                      int vb, int G, int R, int dtype);
void oracle_cache_free(oracle_cache* c);

/* Element counts of the arrays above (for the Python binding). */
size_t oracle_cache_len(const oracle_cache* c, int which);

/* Appends n tokens ([B][H][n][D] raw 16-bit values) one token at a time:
 * before each token, a full window is packed ([G] item 3 of "The Three
 * Structural Innovations of KIVI"; [S] residual length R).
 * Returns 0, or -1 if the capacity would be exceeded (state unchanged). */
int oracle_cache_append(oracle_cache* c, const uint16_t* k, const uint16_t* v,
                        int n);

/* Packs the window when it holds exactly R tokens; otherwise no-op. */
void oracle_cache_flush(oracle_cache* c);

/* Decode attention in binary64 for all B*Hq query heads ([E] "Component 1":
 * each generated token reads the whole cache; [A] abstract).
 * q: raw 16-bit [B][Hq][D]; out: [B][Hq][D] binary64.
 * Returns 0, or -1 if the cache is empty or Hq is not a multiple of H. */
int oracle_decode_attn(const oracle_cache* c, const uint16_t* q, int Hq,
                       double softmax_scale, double* out);

/* Number of OpenMP threads the parallel loops use. */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_ORACLE_H_ */
