// Host-side driver for the sanitizer test: exercises every planner, size
// function and argument check of the C ABI with valid, edge and invalid
// inputs, on the host only. It is linked against host-only objects of the
// library built with AddressSanitizer and UndefinedBehaviorSanitizer, so an
// out-of-bounds access, a signed overflow or a misaligned load in the host
// code aborts the run. No argument below passes validation with a real
// device pointer: every pointer is either null or a never-dereferenced
// placeholder, and each call either fails its host checks or returns
// FA_ERR_HIP (no device, no device code in these objects).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <limits.h>
#include <random>
#include <vector>

#include "fa.h"

static int g_fail = 0;
#define EXPECT(c)                                                              \
  do {                                                                         \
    if (!(c)) {                                                                \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);          \
      ++g_fail;                                                                \
    }                                                                          \
  } while (0)

static void* const P = (void*)(uintptr_t)0x10000;   // placeholder, never dereferenced

static void decode_plans(std::mt19937& rng) {
  const int dims[] = {64, 128, 256, 96, 0, -1};
  for (int it = 0; it < 4000; ++it) {
    const int batch = 1 + (int)(rng() % 70);
    std::vector<int32_t> lens(batch);
    for (auto& L : lens) {
      switch (rng() % 8) {
        case 0: L = 1; break;
        case 1: L = (int32_t)(rng() % 64); break;                      // includes 0 (invalid)
        case 2: L = INT_MAX - (int32_t)(rng() % 3); break;              // extreme
        case 3: L = -(int32_t)(rng() % 5); break;                       // invalid
        default: L = 1 + (int32_t)(rng() % 40000); break;
      }
    }
    const int hkv = 1 + (int)(rng() % 16), group = 1 + (int)(rng() % 9);
    const int hq = (rng() % 10) ? hkv * group : hkv * group + 1;        // sometimes indivisible
    const int d = dims[rng() % 6];
    const int cus = (rng() % 10) ? 256 : (int)(rng() % 3) - 1;
    int sl = -7, ms = -7;
    const int st = fa_decode_plan(lens.data(), batch, hq, hkv, d, cus, &sl, &ms);
    if (st == FA_OK) {
      int64_t mx = 0;
      for (int32_t L : lens) mx = L > mx ? L : mx;
      if (!(sl >= 16 && sl % 16 == 0 && ms >= 1)) fprintf(stderr, "plan b=%d hq=%d hkv=%d d=%d cus=%d -> sl=%d ms=%d\n", batch, hq, hkv, d, cus, sl, ms);
      EXPECT(sl >= 16 && sl % 16 == 0 && ms >= 1);
      EXPECT((int64_t)sl * ms >= mx);
      EXPECT(fa_decode_fused_waves(batch, hq, hkv, d, ms) >= 1);
      (void)fa_decode_fused_workspace_size(batch, hq, hkv, d, ms);
    }
  }
  int sl, ms;
  EXPECT(fa_decode_plan(nullptr, 3, 8, 2, 128, 256, &sl, &ms) != FA_OK);
  int32_t one = 5;
  EXPECT(fa_decode_plan(&one, 1, 8, 2, 128, 256, nullptr, &ms) != FA_OK);
  EXPECT(fa_decode_plan(&one, 0, 8, 2, 128, 256, &sl, &ms) != FA_OK);
}

static void split_plans(std::mt19937& rng) {
  for (int it = 0; it < 1500; ++it) {
    const int batch = (rng() % 20) ? 1 + (int)(rng() % 4) : (int)(rng() % 3) - 1;
    const int sq = (rng() % 15) ? 1 + (int)(rng() % 20000) : (int)(rng() % 3) - 1;
    const int skv = sq + ((rng() % 3) ? 0 : (int)(rng() % 3000));
    const int hkv = 1 + (int)(rng() % 8), group = 1 + (int)(rng() % 8);
    const int hq = (rng() % 12) ? hkv * group : hkv * group + 1;
    const int d = (rng() % 4 == 0) ? 256 : ((rng() % 2) ? 128 : 64);
    const int causal = (int)(rng() % 2), window = (rng() % 3) ? 0 : (int)(rng() % 5000) - 10;
    const int max_units = (int)(rng() % 600);
    std::vector<uint16_t> units((size_t)max_units);    // exactly max_units entries
    const int n = fa_prefill_split_units(batch, sq, skv, hq, hkv, d, causal, window,
                                         max_units ? units.data() : nullptr, max_units);
    if (n > 0) {
      const int nqb = (sq + 127) / 128;
      for (int i = 0; i < n && i < max_units; ++i) {
        EXPECT((units[i] & 0x3fff) < nqb);
        EXPECT((units[i] >> 14) <= 2);
      }
    }
    (void)fa_prefill_split_workspace_size(batch, sq, hq, d);
    (void)fa_prefill_workspace_size(batch, skv, hkv, d);
  }
  // extremes: the size functions must not overflow
  (void)fa_prefill_workspace_size(INT_MAX, INT_MAX, INT_MAX, 512);
  (void)fa_prefill_split_workspace_size(INT_MAX, INT_MAX, INT_MAX, 512);
  (void)fa_decode_fused_workspace_size(INT_MAX, INT_MAX, 1, 256, INT_MAX);
  (void)fa_decode_fused_waves(INT_MAX, INT_MAX, 1, 256, INT_MAX);
  uint16_t u[4];
  (void)fa_prefill_split_units(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 1, 128, 1, 0, u, 4);
}

static void argument_checks(std::mt19937& rng) {
  // every entry point with one argument broken at a time (or all sizes huge)
  const int64_t big = INT64_MAX / 4;
  for (int it = 0; it < 3000; ++it) {
    const int which = (int)(rng() % 12);
    void* q = (rng() % 8) ? P : nullptr;
    const int64_t s1 = (rng() % 6) ? 4096 : ((rng() % 2) ? -8 : big);
    const int64_t s2 = (rng() % 6) ? 512 : ((rng() % 2) ? 3 : big);
    const int64_t s3 = (rng() % 6) ? 128 : ((rng() % 2) ? 0 : big);
    const int batch = (rng() % 6) ? 2 : ((rng() % 2) ? 0 : INT_MAX);
    const int sq = (rng() % 6) ? 300 : ((rng() % 2) ? -1 : INT_MAX);
    const int hq = (rng() % 6) ? 8 : INT_MAX, hkv = (rng() % 6) ? 2 : 3;
    const int d = (rng() % 5) ? 128 : ((rng() % 2) ? 100 : 1024);
    const int dt = (rng() % 8) ? 1 : 7;
    const float scale = (rng() % 8) ? 0.1f : ((rng() % 2) ? 0.0f : -1.0f);
    const uint64_t wsb = (rng() % 4) ? 0 : UINT64_MAX;   // too small or absurd
    int st = FA_OK;
    switch (which) {
      case 0:
        st = fa_prefill_fwd(q, s1, s2, s3, P, s1, s2, s3, P, s1, s2, s3, (float*)P, s1, s2, s3,
                            (float*)P, nullptr, batch, sq, sq, hq, hkv, d, dt, 1, scale, 0,
                            nullptr, 0, nullptr, P, wsb, nullptr);
        break;
      case 1:
        st = fa_prefill_pack_v(q, s1, s2, s3, batch, sq, hkv, d, dt, P, wsb, nullptr);
        break;
      case 2:
        st = fa_prefill_fwd_packed(q, s1, s2, s3, P, s1, s2, s3, (float*)P, s1, s2, s3,
                                   (float*)P, nullptr, batch, sq, sq == INT_MAX ? sq : sq + 1, hq, hkv, d, dt, 1,
                                   scale, 1, nullptr, -3, nullptr, P, wsb, nullptr);
        break;
      case 3:
        st = fa_prefill_fwd_packed_split(q, s1, s2, s3, P, s1, s2, s3, (float*)P, s1, s2, s3,
                                         (float*)P, nullptr, batch, sq, sq, hq, hkv, d, dt, 1,
                                         scale, 0, nullptr, 0, nullptr, P, wsb, P, wsb, nullptr);
        break;
      case 4:
        st = fa_attn_merge((const float*)q, s1, s2, s3, (const float*)P, nullptr, s1, s2, s3,
                           nullptr, nullptr, batch, sq, hq, d, (float*)P, s1, s2, s3,
                           (float*)P, nullptr);
        break;
      case 5:
        st = fa_decode_split_partial(q, s1, s2, P, P, s2, s3, (const int64_t*)P,
                                     (const int32_t*)P, batch, hq, hkv, d, dt, scale, 24, 0,
                                     (float*)P, (float*)P, nullptr);
        break;
      case 6:
        st = fa_decode_merge_lse((const float*)q, (const float*)P, nullptr, batch, hq, d, 20, 0,
                                 (float*)P, (float*)P, nullptr);
        break;
      case 7:
        st = fa_decode_fused(q, s1, s2, P, P, s2, s3, (const int64_t*)P, (const int32_t*)P,
                             batch, hq, hkv, d, dt, scale, 32, 4, (float*)P, (float*)P, P, wsb,
                             nullptr);
        break;
      case 8:
        st = fa_decode_fused_noalloc(q, s1, s2, P, P, s2, s3, (const int64_t*)P,
                                     (const int32_t*)P, batch, hq, hkv, d, dt, scale, 32,
                                     (rng() % 3) ? 4 : INT_MAX, nullptr, (float*)P, nullptr);
        break;
      default: {
        const int s = (int)(rng() % 9) - 2;
        const char* str = fa_status_string(s);
        EXPECT(str != nullptr && strlen(str) > 0);
        break;
      }
    }
    if (which <= 8) {
      EXPECT(st != FA_OK);   // something is always broken, or the device is absent
      const char* e = fa_last_error();
      EXPECT(e != nullptr);
      (void)strlen(e);
    }
  }
}

int main() {
  std::mt19937 rng(12345);
  decode_plans(rng);
  split_plans(rng);
  argument_checks(rng);
  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
