/* oracle_driver.c - runs the C oracle (oracle/kivi_oracle.c) through every
 * entry point on small seeded inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_host_sanitized.py).  Checks the
 * cache invariants on the way; exits non-zero on a failed check. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/kivi_oracle.h"

#define CHECK(c)                                                           \
  do {                                                                     \
    if (!(c)) {                                                            \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      exit(1);                                                             \
    }                                                                      \
  } while (0)

static uint64_t rng = 88172645463325252ull;
static double uniform(void) { /* xorshift64, in [0, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0;
}

static uint16_t f16_of(double x) { return oracle_f32_to_f16((float)x); }

static void fill(uint16_t* a, size_t n, double amp) {
  for (size_t i = 0; i < n; ++i) a[i] = f16_of((uniform() - 0.5) * amp);
}

int main(void) {
  /* quantizer: every code within range, dequantization within the bound */
  for (int it = 0; it < 2000; ++it) {
    float x[64];
    uint8_t codes[64];
    uint16_t s, z;
    const int n = it % 2 ? 32 : 64, bits = it % 3 ? 2 : 4;
    const double amp = it % 7 == 0 ? 0.0 : pow(2.0, (double)(it % 37) - 20.0);
    for (int i = 0; i < n; ++i) x[i] = oracle_f16_to_f32(f16_of((uniform() - 0.5) * amp));
    oracle_quantize_group(x, n, bits, codes, &s, &z);
    for (int i = 0; i < n; ++i) {
      CHECK(codes[i] < (1 << bits));
      CHECK(isfinite(oracle_dequant(codes[i], s, z)));
    }
  }
  /* caches of every bit pair, group size and dtype: appends of random sizes
   * across flushes, the invariants, decode attention */
  const int cfgs[][4] = {{2, 2, 32, 0}, {4, 2, 64, 1}, {2, 4, 32, 1}, {4, 4, 64, 0}};
  for (int c = 0; c < 4; ++c) {
    oracle_cache oc;
    const int B = 2, H = 2, D = 128, Tmax = 700, R = cfgs[c][2] * 2;
    CHECK(oracle_cache_init(&oc, B, H, D, Tmax, cfgs[c][0], cfgs[c][1], cfgs[c][2], R, cfgs[c][3]) == 0);
    uint16_t* k = malloc(sizeof(uint16_t) * B * H * 300 * D);
    uint16_t* v = malloc(sizeof(uint16_t) * B * H * 300 * D);
    uint16_t q[2 * 8 * 128];
    double out[2 * 8 * 128];
    int T = 0;
    while (T < Tmax) {
      int n = 1 + (int)(uniform() * 299);
      if (T + n > Tmax) n = Tmax - T;
      fill(k, (size_t)B * H * n * D, 8.0);
      fill(v, (size_t)B * H * n * D, 8.0);
      CHECK(oracle_cache_append(&oc, k, v, n) == 0);
      T += n;
      CHECK(oc.n_quant + oc.n_resid == T && oc.n_resid >= 1 && oc.n_resid <= R && oc.n_quant % R == 0);
      fill(q, sizeof q / sizeof q[0], 2.0);
      CHECK(oracle_decode_attn(&oc, q, 8, 0.0883883476, out) == 0);
      for (size_t i = 0; i < sizeof out / sizeof out[0]; ++i) CHECK(isfinite(out[i]));
    }
    CHECK(oracle_cache_append(&oc, k, v, 1) == -1); /* capacity: state unchanged */
    CHECK(oc.n_quant + oc.n_resid == Tmax);
    oracle_cache_flush(&oc);
    CHECK(oracle_decode_attn(&oc, q, 3, 0.1, out) == -1); /* 3 query heads over 2 kv heads */
    for (int w = 0; w < 8; ++w) CHECK(oracle_cache_len(&oc, w) > 0);
    free(k);
    free(v);
    oracle_cache_free(&oc);
  }
  printf("oracle driver: ok (%d threads)\n", oracle_num_threads());
  return 0;
}
