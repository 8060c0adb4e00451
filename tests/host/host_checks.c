/* Host-only checks of the library's argument validation, capacity arithmetic
 * and workspace sizing, for a build of the library whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Nothing here launches a
 * kernel or needs a GPU: every call either returns before any launch or only
 * computes sizes.  Exit status 0 when every expectation holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;

#define EXPECT(cond, ...)                 \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      ++failures;                         \
    }                                     \
  } while (0)

static moe_config cfg(int64_t T, int d, int E, int k, int F, double cf) {
  moe_config c;
  memset(&c, 0, sizeof c);
  c.T = T;
  c.d = d;
  c.E = E;
  c.k = k;
  c.d_ff = F;
  c.capacity_factor = cf;
  c.renormalize = -1;
  c.score = MOE_SOFTMAX;
  c.act = MOE_GELU;
  c.dtype = MOE_BF16;
  return c;
}

int main(void) {
  /* the five layer shapes: valid, capacities as the formula gives */
  struct { int64_t T; int d, E, k, F, act, score, n_sh, F_sh; double cf; int64_t C; } ok[] = {
      {64, 32, 4, 2, 64, MOE_GELU, MOE_SOFTMAX, 0, 0, 1.25, 40},
      {4096, 1024, 16, 1, 4096, MOE_GELU, MOE_SOFTMAX, 0, 0, 1.0, 256},
      {8192, 4096, 8, 2, 14336, MOE_SWIGLU, MOE_SOFTMAX, 0, 0, 1.25, 2560},
      {16384, 1024, 64, 6, 512, MOE_GELU, MOE_SOFTMAX, 2, 512, 1.25, 1920},
      {65536, 2048, 128, 8, 1408, MOE_SWIGLU, MOE_SIGMOID, 0, 0, 1.0, 4096},
  };
  for (size_t i = 0; i < sizeof ok / sizeof ok[0]; ++i) {
    moe_config c = cfg(ok[i].T, ok[i].d, ok[i].E, ok[i].k, ok[i].F, ok[i].cf);
    c.act = ok[i].act;
    c.score = ok[i].score;
    c.n_shared = ok[i].n_sh;
    c.d_ff_shared = ok[i].F_sh;
    c.dtype = i == 0 ? MOE_F32 : MOE_BF16;
    int64_t C = -1;
    EXPECT(moe_validate(&c, &C) == MOE_OK && C == ok[i].C, "shape %zu: capacity %lld", i, (long long)C);
    EXPECT(moe_workspace_bytes(&c) > 0 && moe_workspace_bytes(&c) % 256 == 0, "shape %zu: workspace", i);
    for (int mode = 0; mode < 4; ++mode) {
      moe_config m = c;
      m.dropless = mode == 1;
      m.routing = mode == 2 ? MOE_EXPERT_CHOICE : MOE_TOKEN_CHOICE;
      m.priority = mode == 3 ? MOE_SCORE_PRIORITY : MOE_RANK_MAJOR;
      EXPECT(moe_validate(&m, NULL) == MOE_OK, "shape %zu mode %d", i, mode);
      EXPECT(moe_workspace_bytes(&m) > 0, "shape %zu mode %d: workspace", i, mode);
      if (m.dtype == MOE_BF16) EXPECT(moe_backward_workspace_bytes(&m) > 0, "shape %zu mode %d: backward", i, mode);
    }
  }

  /* invalid configurations: refused, with a message, and size queries give 0 */
  const double huge[] = {0.5, NAN, INFINITY, 1e300, 1e9};
  for (size_t i = 0; i < sizeof huge / sizeof huge[0]; ++i) {
    moe_config c = cfg(4096, 1024, 16, 2, 4096, huge[i]);
    int64_t C = 0;
    EXPECT(moe_validate(&c, &C) == MOE_EINVAL, "cf %g accepted (C %lld)", huge[i], (long long)C);
    EXPECT(strlen(moe_last_error()) > 0, "cf %g: no message", huge[i]);
    EXPECT(moe_workspace_bytes(&c) == 0, "cf %g: workspace", huge[i]);
    EXPECT(moe_backward_workspace_bytes(&c) == 0, "cf %g: backward workspace", huge[i]);
  }
  struct { int64_t T; int d, E, k, F; } bad[] = {
      {-1, 64, 4, 2, 64}, {64, 12, 4, 2, 64}, {64, 64, 257, 2, 64}, {64, 64, 4, 0, 64}, {64, 64, 4, 5, 64},
      {64, 64, 64, 33, 64}, {64, 64, 4, 2, 20}, {(int64_t)1 << 29, 64, 8, 4, 64},
  };
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    moe_config c = cfg(bad[i].T, bad[i].d, bad[i].E, bad[i].k, bad[i].F, 1.25);
    EXPECT(moe_validate(&c, NULL) == MOE_EINVAL, "bad shape %zu accepted", i);
  }
  {
    moe_config c = cfg(64, 64, 4, 2, 64, 1.25);
    c.routing = MOE_EXPERT_CHOICE;
    c.dropless = 1;
    EXPECT(moe_validate(&c, NULL) == MOE_EINVAL, "expert choice + dropless accepted");
    c = cfg(64, 64, 4, 2, 64, 1.25);
    c.dtype = MOE_F32;
    c.save_preact = 1;
    EXPECT(moe_validate(&c, NULL) == MOE_EINVAL, "float32 save_preact accepted");
    c = cfg(64, 64, 4, 2, 64, 0.5);
    c.capacity_override = 7;
    int64_t C = 0;
    EXPECT(moe_validate(&c, &C) == MOE_OK && C == 7, "explicit capacity");
  }

  /* entry points refuse NULL or misaligned arguments before any launch */
  {
    moe_config c = cfg(1000, 256, 8, 2, 512, 1.25);
    char buf[64];
    void* odd = buf + 1;
    EXPECT(moe_route(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == MOE_EINVAL,
           "route with NULL outputs");
    EXPECT(moe_dispatch(&c, NULL, (const int32_t*)odd, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == MOE_EINVAL,
           "dispatch with a misaligned idx");
    EXPECT(moe_forward(&c, NULL, NULL, NULL, NULL, NULL) == MOE_EINVAL, "forward with NULL weights");
    moe_weights w;
    moe_outputs o;
    memset(&w, 0, sizeof w);
    memset(&o, 0, sizeof o);
    void* ev[3] = {0, 0, 0};
    EXPECT(moe_forward_events(&c, &w, NULL, &o, NULL, NULL, ev, 3) == MOE_EINVAL, "forward_events with 3 events");
    /* the fixed-scratch dispatch refuses a configuration needing more scratch */
    moe_config big = cfg(200000, 64, 256, 8, 64, 1.25);
    void* p = (void*)(uintptr_t)(1 << 20);
    EXPECT(moe_dispatch_noalloc(&big, NULL, (const int32_t*)p, (int32_t*)p, (uint8_t*)p, (int32_t*)p, NULL, NULL,
                                NULL) == MOE_EINVAL,
           "noalloc dispatch beyond its scratch");
    EXPECT(strstr(moe_last_error(), "scratch") != NULL, "noalloc message");
  }

  if (failures) fprintf(stderr, "%d failures\n", failures);
  else printf("host checks passed\n");
  return failures ? 1 : 0;
}
