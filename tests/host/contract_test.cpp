// contract_test.cpp - the error contract of the C ABI (include/kivi.h),
// exercised on the host state machine with the kernel launchers and HIP
// queries stubbed (stub_launch.cpp).  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py; exits non-zero
// on the first failed check.
//
// Checked: a failed launch returns KIVI_ERR_HIP and poisons the handle
// (later calls return KIVI_ERR_HIP); a failed device query returns
// KIVI_ERR_HIP before anything is enqueued and leaves the cache unchanged
// and usable; the fused decode step plans the state after its append before
// its first launch; launch arguments follow the window rules; a reused
// decode plan equals a fresh one.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/kivi.h"

extern "C" {
void stub_reset(void);
void stub_fail_launch(int n);
void stub_device(int ok, int cus);
int stub_launches(void);
int stub_device_calls(void);
void stub_launch(int i, int* f);
}

namespace {
int g_checks = 0;
#define CHECK(cond)                                                                       \
  do {                                                                                    \
    ++g_checks;                                                                           \
    if (!(cond)) {                                                                        \
      std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, __LINE__, \
                   #cond, kivi_last_error_message());                                     \
      std::exit(1);                                                                       \
    }                                                                                     \
  } while (0)

enum { KIND, NBLK, DST_BLK0, R_COUNT, R_DST, RAGGED, NQ, NR, NSPLIT, NSPLIT_PACKED, HG, FUSED };

void* const kDev = reinterpret_cast<void*>(uintptr_t{0x7f0000000000});  // never dereferenced
void* const kIn = reinterpret_cast<void*>(uintptr_t{0x7f1000000000});
void* const kWs = reinterpret_cast<void*>(uintptr_t{0x7f2000000000});

kivi_config config(int batch = 2, int heads = 2, int max_tokens = 2000) {
  kivi_config c{};
  c.batch = batch;
  c.num_kv_heads = heads;
  c.head_dim = 128;
  c.max_tokens = max_tokens;
  c.k_bits = c.v_bits = 2;
  c.group_size = 32;
  c.residual_length = 128;
  c.kv_dtype = KIVI_F16;
  return c;
}

kivi_cache* make(const kivi_config& c) {
  size_t n = 0;
  CHECK(kivi_cache_bytes(&c, &n) == KIVI_OK);
  kivi_cache* h = nullptr;
  CHECK(kivi_cache_create(&c, kDev, n, &h) == KIVI_OK);
  return h;
}

void lengths(kivi_cache* h, int& nq, int& nr) {
  kivi_cache_view v{};
  CHECK(kivi_cache_get_view(h, &v) == KIVI_OK);
  nq = v.n_quant;
  nr = v.n_resid;
}

int field(int i, int f) {
  int v[12];
  stub_launch(i, v);
  return v[f];
}

size_t ws_bytes(kivi_cache* h, int hq) {
  size_t n = 0;
  CHECK(kivi_decode_attn_workspace_bytes(h, hq, &n) == KIVI_OK);
  return n;
}

kivi_status decode(kivi_cache* h, int hq) {
  return kivi_decode_attn(h, kIn, hq, 0.088f, kWs, KIVI_F32, kWs, ws_bytes(h, hq), nullptr);
}

kivi_status step(kivi_cache* h, int hq) {
  return kivi_append_decode_attn(h, kIn, kIn, kIn, hq, 0.088f, kWs, KIVI_F32, kWs, ws_bytes(h, hq), nullptr);
}

void expect_poisoned(kivi_cache* h, int hq) {
  CHECK(kivi_append(h, kIn, kIn, 1, nullptr) == KIVI_ERR_HIP);
  CHECK(kivi_flush_residual(h, nullptr) == KIVI_ERR_HIP);
  CHECK(decode(h, hq) == KIVI_ERR_HIP);
  CHECK(step(h, hq) == KIVI_ERR_HIP);
  CHECK(kivi_cache_reset(h) == KIVI_ERR_HIP);
}

// A bulk append is one pack launch: whole windows from the input, the last
// 1..R tokens into the window.  A failed launch poisons the handle.
void append_launch_and_poison() {
  stub_reset();
  kivi_cache* h = make(config());
  CHECK(kivi_append(h, kIn, kIn, 300, nullptr) == KIVI_OK);
  int nq, nr;
  lengths(h, nq, nr);
  CHECK(nq == 256 && nr == 44);
  CHECK(stub_launches() == 1 && field(0, KIND) == 0 && field(0, NBLK) == 8 && field(0, DST_BLK0) == 0 &&
        field(0, R_COUNT) == 44);
  // 44 + 100 > R: top up the window (copy), pack it, the rest into the window
  stub_fail_launch(1);
  CHECK(kivi_append(h, kIn, kIn, 100, nullptr) == KIVI_ERR_HIP);
  CHECK(stub_launches() == 1);
  expect_poisoned(h, 4);
  CHECK(stub_launches() == 1);  // a poisoned handle launches nothing
  CHECK(kivi_cache_destroy(h) == KIVI_OK);
}

// The window rules in launch arguments: a full window is packed before the
// next token enters, into blocks n_quant / G ..
void window_rules() {
  stub_reset();
  kivi_cache* h = make(config());
  CHECK(kivi_append(h, kIn, kIn, 256, nullptr) == KIVI_OK);  // (128, 128)
  CHECK(kivi_append(h, kIn, kIn, 1, nullptr) == KIVI_OK);    // flush, then the token
  int nq, nr;
  lengths(h, nq, nr);
  CHECK(nq == 256 && nr == 1);
  CHECK(stub_launches() == 3);
  CHECK(field(1, KIND) == 0 && field(1, NBLK) == 4 && field(1, DST_BLK0) == 4 && field(1, R_COUNT) == 0);
  // an empty window takes the token in a pack launch with no block to pack
  CHECK(field(2, KIND) == 0 && field(2, NBLK) == 0 && field(2, R_COUNT) == 1 && field(2, R_DST) == 0);
  CHECK(kivi_flush_residual(h, nullptr) == KIVI_OK && stub_launches() == 3);  // window not full: no-op
  CHECK(kivi_cache_destroy(h) == KIVI_OK);
}

// A failed device query: KIVI_ERR_HIP before anything is enqueued, cache
// unchanged and not poisoned; the next call queries again.
void device_query_failure() {
  stub_reset();
  stub_device(0, 0);
  kivi_cache* h = make(config());  // creation does not need the device
  CHECK(kivi_append(h, kIn, kIn, 256, nullptr) == KIVI_OK);
  const int launches = stub_launches();
  CHECK(decode(h, 4) == KIVI_ERR_HIP);
  CHECK(step(h, 4) == KIVI_ERR_HIP);
  CHECK(stub_launches() == launches);
  int nq, nr;
  lengths(h, nq, nr);
  CHECK(nq == 128 && nr == 128);  // the step's flush and token were not counted
  stub_device(1, 256);
  CHECK(step(h, 4) == KIVI_OK);  // flush + decode with the fused append
  lengths(h, nq, nr);
  CHECK(nq == 256 && nr == 1);
  CHECK(stub_launches() == launches + 2);
  CHECK(field(launches, KIND) == 0 && field(launches, DST_BLK0) == 4);
  CHECK(field(launches + 1, KIND) == 2 && field(launches + 1, NQ) == 256 && field(launches + 1, NR) == 1 &&
        field(launches + 1, FUSED) == 1 && field(launches + 1, HG) == 1);
  CHECK(kivi_cache_destroy(h) == KIVI_OK);
}

// The fused step uses the plan of the state after its append: the same
// split counts as an explicit append followed by a decode.
void fused_step_plan() {
  for (int hq : {2, 4, 8, 16, 32}) {
    stub_reset();
    kivi_cache* a = make(config(2, 2, 4000));
    kivi_cache* b = make(config(2, 2, 4000));
    CHECK(kivi_append(a, kIn, kIn, 3000, nullptr) == KIVI_OK);
    CHECK(kivi_append(b, kIn, kIn, 3000, nullptr) == KIVI_OK);
    for (int t = 0; t < 200; ++t) {  // crosses a window flush
      int n0 = stub_launches();
      CHECK(step(a, hq) == KIVI_OK);
      const int da = stub_launches() - 1;
      CHECK(field(da, KIND) == 2);
      n0 = stub_launches();
      CHECK(kivi_append(b, kIn, kIn, 1, nullptr) == KIVI_OK);
      CHECK(decode(b, hq) == KIVI_OK);
      const int db = stub_launches() - 1;
      CHECK(field(db, KIND) == 2 && field(da, NQ) == field(db, NQ) && field(da, NR) == field(db, NR));
      CHECK(field(da, NSPLIT) == field(db, NSPLIT) && field(da, NSPLIT_PACKED) == field(db, NSPLIT_PACKED));
      CHECK(field(da, FUSED) == 1 && field(db, FUSED) == 0);
      // 2 kv heads: 16 query heads per kv head take 2 head groups of 8
      CHECK(field(da, HG) == (hq / 2 > 8 ? hq / 16 : 1) && field(db, HG) == field(da, HG));
      (void)n0;
    }
    CHECK(kivi_cache_destroy(a) == KIVI_OK);
    CHECK(kivi_cache_destroy(b) == KIVI_OK);
  }
}

// Failures inside the fused step: the flush launch and the decode launch (4
// and 8 query heads per kv head).
void fused_step_failures() {
  for (int fail_at : {1, 2}) {
    stub_reset();
    kivi_cache* h = make(config());
    CHECK(kivi_append(h, kIn, kIn, 256, nullptr) == KIVI_OK);  // full window: the step flushes
    stub_fail_launch(fail_at);
    CHECK(step(h, 4) == KIVI_ERR_HIP);
    expect_poisoned(h, 4);
    CHECK(kivi_cache_destroy(h) == KIVI_OK);
  }
  {
    // window not full, 8 query heads per kv head: the decode launch alone
    stub_reset();
    kivi_cache* h = make(config());
    CHECK(kivi_append(h, kIn, kIn, 200, nullptr) == KIVI_OK);
    const int launches = stub_launches();
    stub_fail_launch(1);
    CHECK(step(h, 16) == KIVI_ERR_HIP);
    CHECK(stub_launches() == launches);
    expect_poisoned(h, 16);
    CHECK(kivi_cache_destroy(h) == KIVI_OK);
  }
}

// Sequences of different lengths: a failure in any phase of a ragged append
// poisons the handle; lengths follow the per-sequence rules otherwise.
void ragged_paths() {
  stub_reset();
  kivi_cache* h = make(config(3, 2, 3000));
  const int32_t n[3] = {300, 0, 129};
  CHECK(kivi_append_varlen(h, kIn, kIn, n, 300, nullptr) == KIVI_OK);
  int32_t nq[3], nr[3];
  CHECK(kivi_cache_get_lengths(h, nq, nr) == KIVI_OK);
  CHECK(nq[0] == 256 && nr[0] == 44 && nq[1] == 0 && nr[1] == 0 && nq[2] == 128 && nr[2] == 1);
  kivi_cache_view v{};
  CHECK(kivi_cache_get_view(h, &v) == KIVI_OK && v.n_quant == -1 && v.n_resid == -1);
  CHECK(step(h, 4) == KIVI_OK);
  CHECK(kivi_cache_get_lengths(h, nq, nr) == KIVI_OK);
  CHECK(nr[0] == 45 && nr[1] == 1 && nr[2] == 2);
  for (int fail_at : {1, 2, 3}) {
    stub_reset();
    kivi_cache* g = make(config(3, 2, 3000));
    CHECK(kivi_append_varlen(g, kIn, kIn, n, 300, nullptr) == KIVI_OK);
    const int32_t m[3] = {100, 200, 127};  // every phase: window top-up, packs, copies
    stub_fail_launch(fail_at);
    CHECK(kivi_append_varlen(g, kIn, kIn, m, 200, nullptr) == KIVI_ERR_HIP);
    expect_poisoned(g, 4);
    CHECK(kivi_cache_destroy(g) == KIVI_OK);
  }
  CHECK(kivi_cache_destroy(h) == KIVI_OK);
}
// The decode plan is reused while its inputs are unchanged: over fused
// steps of sequences of different lengths (windows flushing at different
// steps, a forced split count set and cleared, the head ratio changing), every
// launch's split counts equal those a fresh cache plans for the same lengths.
// With 2 compute units no ragged grid fits one round, and the plan then
// depends on every sequence's length, not only the longest.
void plan_reuse() {
  for (int cus : {256, 2}) {
  stub_reset();
  stub_device(1, cus);
  const kivi_config cf = config(5, 2, 6000);
  kivi_cache* a = make(cf);
  const int32_t n[5] = {3000, 1200, 5000, 0, 2500};
  CHECK(kivi_append_varlen(a, kIn, kIn, n, 5000, nullptr) == KIVI_OK);
  for (int t = 0; t < 300; ++t) {
    const int hq = t < 150 ? 32 : (t < 220 ? 2 : 8);
    if (t == 100) CHECK(kivi_set_decode_splits(a, 3) == KIVI_OK);
    if (t == 120) CHECK(kivi_set_decode_splits(a, 0) == KIVI_OK);
    CHECK(step(a, hq) == KIVI_OK);
    const int da = stub_launches() - 1;
    CHECK(field(da, KIND) == 2 && field(da, FUSED) == 1);
    int32_t nq[5], nr[5];
    CHECK(kivi_cache_get_lengths(a, nq, nr) == KIVI_OK);
    kivi_cache* b = make(cf);
    CHECK(kivi_cache_set_lengths(b, nq, nr) == KIVI_OK);
    if (t >= 100 && t < 120) CHECK(kivi_set_decode_splits(b, 3) == KIVI_OK);
    CHECK(decode(b, hq) == KIVI_OK);
    const int db = stub_launches() - 1;
    CHECK(field(db, KIND) == 2 && field(db, RAGGED) == field(da, RAGGED));
    CHECK(field(da, NSPLIT) == field(db, NSPLIT) && field(da, NSPLIT_PACKED) == field(db, NSPLIT_PACKED));
    CHECK(field(da, HG) == field(db, HG));
    CHECK(kivi_cache_destroy(b) == KIVI_OK);
  }
  CHECK(kivi_cache_destroy(a) == KIVI_OK);
  }
}

// The largest forced split count: 1020 packed streams in 255 splits of one
// step, plus the window's partial: 256, the most the merge takes.
void most_splits() {
  stub_reset();
  kivi_cache* h = make(config(1, 2, 32700));
  CHECK(kivi_append(h, kIn, kIn, 32700, nullptr) == KIVI_OK);
  int nq, nr;
  lengths(h, nq, nr);
  CHECK(nq == 32640 && nr == 60);
  CHECK(kivi_set_decode_splits(h, 1000000) == KIVI_OK);
  CHECK(decode(h, 8) == KIVI_OK);
  const int d = stub_launches() - 1;
  CHECK(field(d, KIND) == 2 && field(d, NSPLIT) == 256 && field(d, NSPLIT_PACKED) == 255);
  CHECK(kivi_cache_destroy(h) == KIVI_OK);
}

// Declared lengths (a restored snapshot): validated per sequence, no launch.
void set_lengths_rules() {
  stub_reset();
  kivi_cache* h = make(config(2, 2, 1000));
  const int32_t q1[2] = {256, 128}, r1[2] = {5, 128};
  CHECK(kivi_cache_set_lengths(h, q1, r1) == KIVI_OK);
  int32_t nq[2], nr[2];
  CHECK(kivi_cache_get_lengths(h, nq, nr) == KIVI_OK);
  CHECK(nq[0] == 256 && nr[0] == 5 && nq[1] == 128 && nr[1] == 128);
  int v_nq, v_nr;
  lengths(h, v_nq, v_nr);
  CHECK(v_nq == -1 && v_nr == -1);
  const int32_t bad[3][2][2] = {{{100, 0}, {0, 0}}, {{0, 0}, {129, 0}}, {{896, 0}, {128, 0}}};
  for (const auto& b : bad) {
    CHECK(kivi_cache_set_lengths(h, b[0], b[1]) == KIVI_ERR_INVALID_ARG);
    CHECK(kivi_cache_get_lengths(h, nq, nr) == KIVI_OK && nq[0] == 256 && nr[0] == 5);
  }
  const int32_t q2[2] = {256, 256}, r2[2] = {0, 0};  // equal lengths: the uniform state
  CHECK(kivi_cache_set_lengths(h, q2, r2) == KIVI_OK);
  lengths(h, v_nq, v_nr);
  CHECK(v_nq == 256 && v_nr == 0);
  CHECK(kivi_append(h, kIn, kIn, 1, nullptr) == KIVI_OK);  // an empty window takes the token
  lengths(h, v_nq, v_nr);
  CHECK(v_nq == 256 && v_nr == 1);
  CHECK(stub_launches() == 1);
  CHECK(kivi_set_timing_events(h, kDev, nullptr) == KIVI_ERR_INVALID_ARG);
  CHECK(kivi_set_timing_events(h, nullptr, nullptr) == KIVI_OK);
  CHECK(kivi_cache_destroy(h) == KIVI_OK);
}
}  // namespace

int main() {
  append_launch_and_poison();
  window_rules();
  device_query_failure();
  fused_step_plan();
  fused_step_failures();
  ragged_paths();
  plan_reuse();
  most_splits();
  set_lengths_rules();
  std::printf("contract: %d checks passed\n", g_checks);
  return 0;
}
