/*
 * kivi_oracle.c - plain, slow CPU oracle of the KIVI hot path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the package smoke check and
 * the CPU-baseline leg of the benchmark; never by the product path.
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 *
 * Page keys used in the citations:
 *   [G] "KIVI: Asymmetric 2-Bit KV Cache Quantization Guide"
 *   [S] "KV cache quantization with KIVI INT2 setup guide"
 *   [E] "KV-Cache Quantization: I Ran the Experiments So You Don't Have To"
 *   [A] "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 */
#include "kivi_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- floats */

float oracle_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return (float)(sign ? -v : v);
}

float oracle_bf16_to_f32(uint16_t h) {
  /* bfloat16 is the upper half of a binary32 word. */
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

uint16_t oracle_f32_to_f16(float f) {
  if (isnan(f)) return 0x7e00;
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  double a = fabs((double)f);
  if (a >= 65520.0) return sign | 0x7c00; /* rounds to infinity */
  if (a == 0.0) return sign;
  /* quantum of the binary16 grid around a */
  int E;
  frexp(a, &E); /* a = m * 2^E, m in [0.5, 1) => a in [2^(E-1), 2^E) */
  int e = E - 1;
  double quantum = (e < -14) ? ldexp(1.0, -24) : ldexp(1.0, e - 10);
  double n = rint(a / quantum); /* exact quotient, ties to even */
  double r = n * quantum;       /* rounded magnitude, exact */
  if (r < ldexp(1.0, -14)) {
    return sign | (uint16_t)(r / ldexp(1.0, -24)); /* subnormal (or 0) */
  }
  frexp(r, &E);
  e = E - 1;
  int mant = (int)(r / ldexp(1.0, e - 10)) - 1024;
  return sign | (uint16_t)(((e + 15) << 10) | mant);
}

static float load_elem(uint16_t raw, int dtype) {
  return dtype == 0 ? oracle_f16_to_f32(raw) : oracle_bf16_to_f32(raw);
}

/* ------------------------------------------------------------- quantizer */

/* [G] "Step 1": per group, min and max give the scale (max - min) / qmax and
 * every value is rounded (half to even, like torch.round) to an integer code
 * in [0, qmax].  The zero-point is the group minimum in floating point, so
 * the code of the minimum is 0, the code of the maximum is qmax and a
 * constant group has scale 0 and is reproduced exactly.  Each arithmetic
 * step below is one binary32 operation. */
void oracle_quantize_group(const float* x, int n, int bits, uint8_t* codes,
                           uint16_t* scale_f16, uint16_t* zero_f16) {
  const float qmax = (float)((1 << bits) - 1);
  float mn = x[0], mx = x[0];
  for (int j = 1; j < n; ++j) {
    if (x[j] < mn) mn = x[j];
    if (x[j] > mx) mx = x[j];
  }
  float range = mx - mn;
  float s = range / qmax;
  for (int j = 0; j < n; ++j) {
    if (s == 0.0f) {
      codes[j] = 0;
      continue;
    }
    float d = x[j] - mn;
    float y = d / s;
    float c = rintf(y); /* default rounding mode: nearest, ties to even */
    if (c < 0.0f) c = 0.0f;
    if (c > qmax) c = qmax;
    codes[j] = (uint8_t)c;
  }
  *scale_f16 = (s == 0.0f) ? 0 : oracle_f32_to_f16(s);
  *zero_f16 = (mn == 0.0f) ? 0 : oracle_f32_to_f16(mn);
}

/* [G] "Step 2": value = code * scale + zero (floating zero-point form). */
double oracle_dequant(int code, uint16_t scale_f16, uint16_t zero_f16) {
  return (double)code * (double)oracle_f16_to_f32(scale_f16) +
         (double)oracle_f16_to_f32(zero_f16);
}

/* ---------------------------------------------------------------- layout */

/* Bit offset of code number i inside its 32-bit word: even codes fill the low
 * half-word and odd codes the high half-word, each in increasing order. */
static int code_bit_offset(int i, int bits) { return bits * (i / 2) + 16 * (i % 2); }

static size_t k_words_per_token(const oracle_cache* c) { return (size_t)c->D * c->kb / 32; }
static size_t v_words_per_channel(const oracle_cache* c) { return (size_t)c->G * c->vb / 32; }

size_t oracle_cache_len(const oracle_cache* c, int which) {
  size_t U = (size_t)c->B * c->H;
  switch (which) {
    case 0: return U * c->cap * k_words_per_token(c);                 /* k_codes */
    case 1: return U * c->nb * c->D;                                  /* k_scale */
    case 2: return U * c->nb * c->D;                                  /* k_zero */
    case 3: return U * c->nb * c->D * v_words_per_channel(c);         /* v_codes */
    case 4: return U * c->nb * (c->D / c->G) * c->G;                  /* v_scale */
    case 5: return U * c->nb * (c->D / c->G) * c->G;                  /* v_zero */
    case 6: return U * c->R * c->D;                                   /* k_resid */
    case 7: return U * c->R * c->D;                                   /* v_resid */
    default: return 0;
  }
}

int oracle_cache_init(oracle_cache* c, int B, int H, int D, int T_max, int kb,
                      int vb, int G, int R, int dtype) {
  memset(c, 0, sizeof *c);
  if (B < 1 || H < 1 || G < 2 || D < G || D % G || R < G || R % G ||
      T_max < 1 || (kb != 2 && kb != 4) || (vb != 2 && vb != 4) ||
      (dtype != 0 && dtype != 1) || (D * kb) % 32 || (G * vb) % 32 ||
      G > 1024 || D > 1024)
    return -1;
  c->B = B; c->H = H; c->D = D; c->T_max = T_max; c->kb = kb; c->vb = vb;
  c->G = G; c->R = R; c->dtype = dtype;
  c->cap = ((T_max + R - 1) / R) * R;
  c->nb = c->cap / G;
  c->k_codes = calloc(oracle_cache_len(c, 0), sizeof(uint32_t));
  c->k_scale = calloc(oracle_cache_len(c, 1), sizeof(uint16_t));
  c->k_zero = calloc(oracle_cache_len(c, 2), sizeof(uint16_t));
  c->v_codes = calloc(oracle_cache_len(c, 3), sizeof(uint32_t));
  c->v_scale = calloc(oracle_cache_len(c, 4), sizeof(uint16_t));
  c->v_zero = calloc(oracle_cache_len(c, 5), sizeof(uint16_t));
  c->k_resid = calloc(oracle_cache_len(c, 6), sizeof(uint16_t));
  c->v_resid = calloc(oracle_cache_len(c, 7), sizeof(uint16_t));
  if (!c->k_codes || !c->k_scale || !c->k_zero || !c->v_codes || !c->v_scale ||
      !c->v_zero || !c->k_resid || !c->v_resid) {
    oracle_cache_free(c);
    return -1;
  }
  return 0;
}

void oracle_cache_free(oracle_cache* c) {
  free(c->k_codes); free(c->k_scale); free(c->k_zero);
  free(c->v_codes); free(c->v_scale); free(c->v_zero);
  free(c->k_resid); free(c->v_resid);
  memset(c, 0, sizeof *c);
}

/* ------------------------------------------------------------------ pack */

/* Packs the R tokens of unit u's residual window into token positions
 * n_quant .. n_quant + R - 1.
 * Keys, per channel ([G] item 1 of "The Three Structural Innovations of
 * KIVI"; [S] group size 32): each block of G tokens of one channel is one
 * group.  Values, per token ([G] item 2): each run of G channels of one token
 * is one group. */
static void pack_window_unit(oracle_cache* c, size_t u) {
  const int G = c->G, D = c->D, R = c->R;
  const size_t kw = k_words_per_token(c), vw = v_words_per_channel(c);
  const int Pk = 32 / c->kb, Pv = 32 / c->vb;
  const uint16_t* kres = c->k_resid + u * R * D;
  const uint16_t* vres = c->v_resid + u * R * D;
  float x[1024];
  uint8_t code[1024];
  uint8_t* kc = malloc((size_t)G * D); /* codes of one block, [row][channel] */
  uint8_t* vc = malloc((size_t)G * D);

  for (int blk = 0; blk < R / G; ++blk) {
    const int g = c->n_quant / G + blk; /* global block index */
    /* key groups: channel d, rows 0..G-1 of this block */
    for (int d = 0; d < D; ++d) {
      for (int j = 0; j < G; ++j)
        x[j] = load_elem(kres[(size_t)(blk * G + j) * D + d], c->dtype);
      uint16_t S, Z;
      oracle_quantize_group(x, G, c->kb, code, &S, &Z);
      c->k_scale[(u * c->nb + g) * D + d] = S;
      c->k_zero[(u * c->nb + g) * D + d] = Z;
      for (int j = 0; j < G; ++j) kc[j * D + d] = code[j];
    }
    /* value groups: row j, channels m*G .. m*G+G-1 */
    for (int j = 0; j < G; ++j) {
      for (int m = 0; m < D / G; ++m) {
        for (int i = 0; i < G; ++i)
          x[i] = load_elem(vres[(size_t)(blk * G + j) * D + m * G + i], c->dtype);
        uint16_t S, Z;
        oracle_quantize_group(x, G, c->vb, code, &S, &Z);
        c->v_scale[((u * c->nb + g) * (D / G) + m) * G + j] = S;
        c->v_zero[((u * c->nb + g) * (D / G) + m) * G + j] = Z;
        for (int i = 0; i < G; ++i) vc[j * D + m * G + i] = code[i];
      }
    }
    /* key words: token row t, word w holds channels w*Pk .. w*Pk+Pk-1 */
    for (int j = 0; j < G; ++j) {
      const size_t t = (size_t)g * G + j;
      for (size_t w = 0; w < kw; ++w) {
        uint32_t word = 0;
        for (int i = 0; i < Pk; ++i)
          word |= (uint32_t)kc[j * D + w * Pk + i] << code_bit_offset(i, c->kb);
        c->k_codes[(u * c->cap + t) * kw + w] = word;
      }
    }
    /* value words: word w of channel d in block g holds rows w*Pv ..
     * w*Pv+Pv-1; the D words of one w are stored next to each other */
    for (size_t w = 0; w < vw; ++w) {
      for (int d = 0; d < D; ++d) {
        uint32_t word = 0;
        for (int i = 0; i < Pv; ++i)
          word |= (uint32_t)vc[(w * Pv + i) * D + d] << code_bit_offset(i, c->vb);
        c->v_codes[((u * c->nb + g) * vw + w) * D + d] = word;
      }
    }
  }
  free(kc);
  free(vc);
}

static void pack_window(oracle_cache* c) {
  const long U = (long)c->B * c->H;
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < U; ++u) pack_window_unit(c, (size_t)u);
  c->n_quant += c->R;
  c->n_resid = 0;
}

/* [G] item 3 and "Step 3": new tokens enter the full-precision window; a
 * window that is full is grouped and packed before the next token enters
 * (whole-window flush, so 1 <= n_resid <= R after any append). */
int oracle_cache_append(oracle_cache* c, const uint16_t* k, const uint16_t* v,
                        int n) {
  if (n < 0 || (long)c->n_quant + c->n_resid + n > c->T_max) return -1;
  const long U = (long)c->B * c->H;
  const int D = c->D;
  for (int i = 0; i < n; ++i) {
    if (c->n_resid == c->R) pack_window(c);
    for (long u = 0; u < U; ++u) {
      memcpy(c->k_resid + ((size_t)u * c->R + c->n_resid) * D,
             k + ((size_t)u * n + i) * D, (size_t)D * sizeof(uint16_t));
      memcpy(c->v_resid + ((size_t)u * c->R + c->n_resid) * D,
             v + ((size_t)u * n + i) * D, (size_t)D * sizeof(uint16_t));
    }
    c->n_resid += 1;
  }
  return 0;
}

void oracle_cache_flush(oracle_cache* c) {
  if (c->n_resid == c->R) pack_window(c);
}

/* -------------------------------------------------------------- attention */

/* Dequantized key channel d of token t (t < n_quant) of unit u. */
static double key_hat(const oracle_cache* c, size_t u, int t, int d) {
  const size_t kw = k_words_per_token(c);
  const int Pk = 32 / c->kb;
  uint32_t word = c->k_codes[(u * c->cap + t) * kw + d / Pk];
  int code = (word >> code_bit_offset(d % Pk, c->kb)) & ((1 << c->kb) - 1);
  size_t mi = (u * c->nb + t / c->G) * c->D + d;
  return oracle_dequant(code, c->k_scale[mi], c->k_zero[mi]);
}

/* Dequantized value channel d of token t (t < n_quant) of unit u. */
static double value_hat(const oracle_cache* c, size_t u, int t, int d) {
  const size_t vw = v_words_per_channel(c);
  const int Pv = 32 / c->vb, G = c->G;
  const int g = t / G, j = t % G;
  uint32_t word = c->v_codes[((u * c->nb + g) * vw + j / Pv) * c->D + d];
  int code = (word >> code_bit_offset(j % Pv, c->vb)) & ((1 << c->vb) - 1);
  size_t mi = ((u * c->nb + g) * (c->D / G) + d / G) * G + j;
  return oracle_dequant(code, c->v_scale[mi], c->v_zero[mi]);
}

/* Scaled dot-product attention of one query over all cached tokens:
 * s_t = scale * q . k^_t, p = softmax(s), out = sum_t p_t v^_t, with k^, v^
 * dequantized for packed tokens and taken as stored for window tokens. */
int oracle_decode_attn(const oracle_cache* c, const uint16_t* q, int Hq,
                       double softmax_scale, double* out) {
  const int T = c->n_quant + c->n_resid;
  if (T < 1 || Hq < c->H || Hq % c->H) return -1;
  const int D = c->D, gq = Hq / c->H;
  const long heads = (long)c->B * Hq;
  int fail = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : fail)
  for (long bj = 0; bj < heads; ++bj) {
    const long b = bj / Hq, j = bj % Hq;
    const size_t u = (size_t)b * c->H + (size_t)(j / gq); /* kv head j / gq */
    double* s = malloc(sizeof(double) * T);
    double* qd = malloc(sizeof(double) * D);
    if (!s || !qd) {
      fail = 1;
      free(s); free(qd);
      continue;
    }
    for (int d = 0; d < D; ++d) qd[d] = load_elem(q[bj * D + d], c->dtype);
    for (int t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) {
        double kv = (t < c->n_quant)
                        ? key_hat(c, u, t, d)
                        : load_elem(c->k_resid[(u * c->R + (t - c->n_quant)) * D + d],
                                    c->dtype);
        acc += qd[d] * kv;
      }
      s[t] = softmax_scale * acc;
    }
    double mx = s[0];
    for (int t = 1; t < T; ++t) if (s[t] > mx) mx = s[t];
    double l = 0.0;
    for (int t = 0; t < T; ++t) { s[t] = exp(s[t] - mx); l += s[t]; }
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int t = 0; t < T; ++t) {
        double vv = (t < c->n_quant)
                        ? value_hat(c, u, t, d)
                        : load_elem(c->v_resid[(u * c->R + (t - c->n_quant)) * D + d],
                                    c->dtype);
        acc += s[t] * vv;
      }
      out[bj * D + d] = acc / l;
    }
    free(s);
    free(qd);
  }
  return fail ? -1 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
