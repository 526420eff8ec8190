// Drives the host layer of librkv (argument validation, workspace sizing,
// status strings, the no-op paths below the eviction trigger) with the
// library's sources built for the host only, under AddressSanitizer and
// UndefinedBehaviorSanitizer. Every call here either fails validation or
// takes a documented path that launches nothing, so the fake device pointers
// are never dereferenced and no GPU is needed. Exit status 0 when every
// call returned what include/rkv.h documents; the sanitizers abort on any
// finding.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "rkv.h"

static int failures = 0;
#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    const int got_ = (int)(call);                                                           \
    if (got_ != (int)(want)) {                                                              \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                           \
    }                                                                                       \
  } while (0)

static void* const FAKE = (void*)0x10000;
static void* const FAKE_WS = (void*)0x100000;
static void* at(void* p, uintptr_t off) { return (void*)((uintptr_t)p + off); }

static rkv_params P() {
  rkv_params p;
  memset(&p, 0, sizeof(p));
  p.num_layers = 2;
  p.batch = 2;
  p.num_kv_heads = 2;
  p.group = 4;
  p.head_dim = 128;
  p.capacity = 384;
  p.budget = 256;
  p.buffer = 128;
  p.obs_window = 8;
  p.beta = 2;
  p.lambda = 0.1f;
  p.sim_threshold = 0.5f;
  p.dtype = RKV_BF16;
  return p;
}

static void* layers_[RKV_MAX_LAYERS];
static void* const* layers(int n = 2) {
  for (int i = 0; i < n; ++i) layers_[i] = at(FAKE, 4096u * i);
  return layers_;
}

static float* F(void* p) { return (float*)p; }
static int32_t* I(void* p) { return (int32_t*)p; }

// every entry point on one parameter block that validation rejects with `want`
static void all_reject(const rkv_params& p, rkv_status want) {
  const size_t big = (size_t)1 << 40;
  int32_t ns;
  EXPECT(rkv_score(&p, layers(), FAKE, I(FAKE), 300, F(FAKE), F(FAKE), nullptr, FAKE_WS, big, nullptr), want);
  EXPECT(rkv_select(&p, F(FAKE), F(FAKE), I(FAKE), 300, I(FAKE), nullptr, nullptr, nullptr), want);
  EXPECT(rkv_compact(&p, layers(), layers(), I(FAKE), I(FAKE), 300, nullptr), want);
  ns = 384;
  EXPECT(rkv_evict_step(&p, layers(), layers(), FAKE, I(FAKE), &ns, FAKE_WS, big, nullptr), want);
  EXPECT(ns, 384);
  ns = 384;
  EXPECT(rkv_evict_step_timed(&p, layers(), layers(), FAKE, I(FAKE), &ns, FAKE_WS, big, nullptr, nullptr), want);
  ns = 384;
  EXPECT(rkv_evict_step_holefill(&p, layers(), layers(), FAKE, I(FAKE), I(FAKE), &ns, FAKE_WS, big, nullptr), want);
  EXPECT(rkv_compact_holefill(&p, layers(), layers(), I(FAKE), I(FAKE), I(FAKE), 300, nullptr), want);
  EXPECT(rkv_decode_attention(&p, layers(), layers(), FAKE, I(FAKE), 300, F(FAKE), nullptr, nullptr), want);
  ns = 384;
  EXPECT(rkv_evict_step_captured(&p, layers(), layers(), F(FAKE), I(FAKE), &ns, FAKE_WS, big, nullptr), want);
  ns = 384;
  EXPECT(rkv_evict_step_noalloc(&p, layers(), layers(), FAKE, I(FAKE), &ns, nullptr), want);
  EXPECT(rkv_select_sampled(&p, F(FAKE), F(FAKE), I(FAKE), 300, 8, 10, 1.f, I(FAKE), nullptr), want);
  ns = 384;
  EXPECT(rkv_evict_step_sampled(&p, layers(), layers(), F(FAKE), F(FAKE), I(FAKE), &ns, 8, 10, 1.f, FAKE_WS, big,
                                nullptr),
         want);
  ns = 384;
  EXPECT(rkv_evict_step_sentences(&p, layers(), layers(), FAKE, I(FAKE), &ns, I(FAKE), F(FAKE), I(FAKE), 16, 64, 0.8f,
                                  F(FAKE), FAKE_WS, big, nullptr),
         want);
  EXPECT(rkv_workspace_bytes(&p), 0);
}

static void bad_params() {
  struct Case {
    void (*edit)(rkv_params&);
    rkv_status want;
  } cases[] = {
      {[](rkv_params& p) { p.lambda = 1.5f; }, RKV_ERR_BAD_PARAM},
      {[](rkv_params& p) { p.lambda = NAN; }, RKV_ERR_BAD_PARAM},
      {[](rkv_params& p) { p.sim_threshold = -1.5f; }, RKV_ERR_BAD_PARAM},
      {[](rkv_params& p) { p.beta = -1; }, RKV_ERR_BAD_PARAM},
      {[](rkv_params& p) { p.dtype = 7; }, RKV_ERR_BAD_PARAM},
      {[](rkv_params& p) { p.num_layers = 0; }, RKV_ERR_BAD_SHAPE},
      {[](rkv_params& p) { p.num_layers = RKV_MAX_LAYERS + 1; }, RKV_ERR_BAD_SHAPE},
      {[](rkv_params& p) { p.batch = -5; }, RKV_ERR_BAD_SHAPE},
      {[](rkv_params& p) { p.obs_window = 0; }, RKV_ERR_BAD_SHAPE},
      {[](rkv_params& p) { p.budget = 8; }, RKV_ERR_BAD_SHAPE},
      {[](rkv_params& p) { p.buffer = 0; }, RKV_ERR_BAD_SHAPE},
      {[](rkv_params& p) { p.capacity = 383; }, RKV_ERR_BAD_SHAPE},
      // sums near INT32_MAX must not overflow inside validation
      {[](rkv_params& p) { p.budget = 2147483000; p.buffer = 2147483000; }, RKV_ERR_BAD_SHAPE},
      {[](rkv_params& p) { p.head_dim = 64; }, RKV_ERR_UNSUPPORTED},
      {[](rkv_params& p) { p.capacity = 20000; }, RKV_ERR_UNSUPPORTED},
      {[](rkv_params& p) { p.group = 9; }, RKV_ERR_UNSUPPORTED},
      {[](rkv_params& p) { p.group = 2147483647; }, RKV_ERR_UNSUPPORTED},
      {[](rkv_params& p) { p.batch = 2147483647; p.num_kv_heads = 2147483647; }, RKV_ERR_UNSUPPORTED},
  };
  for (const Case& c : cases) {
    rkv_params p = P();
    c.edit(p);
    all_reject(p, c.want);
  }
  EXPECT(rkv_workspace_bytes(nullptr), 0);
  if (rkv_workspace_keep_offset(nullptr) != SIZE_MAX) {
    fprintf(stderr, "keep offset of NULL params\n");
    ++failures;
  }
  int32_t ns = 384;
  EXPECT(rkv_evict_step(nullptr, layers(), layers(), FAKE, I(FAKE), &ns, FAKE_WS, 1, nullptr), RKV_ERR_NULL_ARG);
}

static void pointers_and_ranges() {
  rkv_params p = P();
  const size_t need = rkv_workspace_bytes(&p), big = (size_t)1 << 40;
  if (need == 0 || need % 256 != 0 || rkv_workspace_keep_offset(&p) >= need) {
    fprintf(stderr, "workspace sizes %zu %zu\n", need, rkv_workspace_keep_offset(&p));
    ++failures;
  }
  void* with_null[2] = {FAKE, nullptr};
  void* misaligned[2] = {at(FAKE, 8), FAKE};
  int32_t ns;
  EXPECT(rkv_score(&p, with_null, FAKE, I(FAKE), 300, F(FAKE), F(FAKE), nullptr, FAKE_WS, big, nullptr),
         RKV_ERR_NULL_ARG);
  EXPECT(rkv_score(&p, misaligned, FAKE, I(FAKE), 300, F(FAKE), F(FAKE), nullptr, FAKE_WS, big, nullptr),
         RKV_ERR_MISALIGNED);
  EXPECT(rkv_score(&p, layers(), at(FAKE, 4), I(FAKE), 300, F(FAKE), F(FAKE), nullptr, FAKE_WS, big, nullptr),
         RKV_ERR_MISALIGNED);
  EXPECT(rkv_score(&p, layers(), FAKE, I(FAKE), 385, F(FAKE), F(FAKE), nullptr, FAKE_WS, need, nullptr),
         RKV_ERR_BAD_SHAPE);
  EXPECT(rkv_score(&p, layers(), FAKE, I(FAKE), -2147483647 - 1, F(FAKE), F(FAKE), nullptr, FAKE_WS, need, nullptr),
         RKV_ERR_BAD_SHAPE);
  EXPECT(rkv_score(&p, layers(), FAKE, I(FAKE), 300, F(FAKE), F(FAKE), nullptr, FAKE_WS, need - 1, nullptr),
         RKV_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(rkv_select(&p, nullptr, F(FAKE), I(FAKE), 300, I(FAKE), nullptr, nullptr, nullptr), RKV_ERR_NULL_ARG);
  EXPECT(rkv_select(&p, F(FAKE), F(FAKE), I(FAKE), 255, I(FAKE), nullptr, nullptr, nullptr), RKV_ERR_BAD_SHAPE);
  EXPECT(rkv_compact(&p, layers(), with_null, I(FAKE), I(FAKE), 300, nullptr), RKV_ERR_NULL_ARG);
  ns = 385;
  EXPECT(rkv_evict_step(&p, layers(), layers(), FAKE, I(FAKE), &ns, FAKE_WS, need, nullptr), RKV_ERR_BAD_SHAPE);
  EXPECT(ns, 385);
  ns = 384;
  EXPECT(rkv_evict_step(&p, layers(), layers(), FAKE, I(FAKE), &ns, FAKE_WS, need - 256, nullptr),
         RKV_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(rkv_evict_step(&p, layers(), layers(), FAKE, I(FAKE), nullptr, FAKE_WS, need, nullptr), RKV_ERR_NULL_ARG);
  // the sampled, sentence, decode and hole-filling argument checks
  EXPECT(rkv_select_sampled(&p, F(FAKE), F(FAKE), I(FAKE), 300, -1, 10, 1.f, I(FAKE), nullptr), RKV_ERR_BAD_PARAM);
  EXPECT(rkv_select_sampled(&p, F(FAKE), F(FAKE), I(FAKE), 300, 8, 10, INFINITY, I(FAKE), nullptr),
         RKV_ERR_BAD_PARAM);
  EXPECT(rkv_sentence_penalty(&p, F(FAKE), I(FAKE), 16, 66, 0.8f, F(FAKE), nullptr), RKV_ERR_BAD_SHAPE);
  EXPECT(rkv_sentence_penalty(&p, F(FAKE), I(FAKE), 2147483647, 2147483647, 0.8f, F(FAKE), nullptr),
         RKV_ERR_BAD_SHAPE);
  EXPECT(rkv_sentence_penalty(&p, F(at(FAKE, 8)), I(FAKE), 16, 64, 0.8f, F(FAKE), nullptr), RKV_ERR_MISALIGNED);
  EXPECT(rkv_decode_attention(&p, layers(), layers(), FAKE, I(FAKE), 385, F(FAKE), nullptr, nullptr),
         RKV_ERR_BAD_SHAPE);
  rkv_params dec = P();
  dec.group = 8;
  dec.capacity = 8000;
  dec.budget = 7000;
  EXPECT(rkv_decode_attention(&dec, layers(), layers(), FAKE, I(FAKE), 6000, F(FAKE), nullptr, nullptr),
         RKV_ERR_UNSUPPORTED);
  EXPECT(rkv_compact_holefill(&p, layers(), layers(), I(FAKE), I(FAKE), I(at(FAKE, 1)), 300, nullptr),
         RKV_ERR_MISALIGNED);
  rkv_params hf = P();
  hf.budget = 12000;
  hf.capacity = 12200;
  ns = 12200;
  EXPECT(rkv_evict_step_holefill(&hf, layers(), layers(), FAKE, I(FAKE), I(FAKE), &ns, FAKE_WS, big, nullptr),
         RKV_ERR_UNSUPPORTED);
  // the allocation-free step: a workspace beyond its built-in array
  rkv_params na = P();
  na.num_layers = 32;
  na.batch = 32;
  na.num_kv_heads = 8;
  na.capacity = 1152;
  na.budget = 1024;
  ns = 1152;
  EXPECT(rkv_evict_step_noalloc(&na, layers(32), layers(32), FAKE, I(FAKE), &ns, nullptr),
         RKV_ERR_WORKSPACE_TOO_SMALL);
}

static void no_launch_paths() {
  rkv_params p = P();
  const size_t need = rkv_workspace_bytes(&p);
  for (int n : {0, 1, 255, 256, 383}) {
    int32_t ns = n;
    EXPECT(rkv_evict_step(&p, layers(), layers(), FAKE, I(FAKE), &ns, FAKE_WS, need, nullptr), RKV_OK);
    EXPECT(ns, n);
    EXPECT(rkv_evict_step_holefill(&p, layers(), layers(), FAKE, I(FAKE), I(FAKE), &ns, FAKE_WS, need, nullptr),
           RKV_OK);
    EXPECT(rkv_evict_step_captured(&p, layers(), layers(), F(FAKE), I(FAKE), &ns, FAKE_WS, need, nullptr), RKV_OK);
    EXPECT(rkv_evict_step_noalloc(&p, layers(), layers(), FAKE, I(FAKE), &ns, nullptr), RKV_OK);
    EXPECT(rkv_evict_step_sampled(&p, layers(), layers(), F(FAKE), F(FAKE), I(FAKE), &ns, 8, 10, 1.f, FAKE_WS, need,
                                  nullptr),
           RKV_OK);
    EXPECT(ns, n);
  }
  for (int n : {0, 100, 256})
    EXPECT(rkv_score(&p, layers(), FAKE, I(FAKE), n, F(FAKE), F(FAKE), nullptr, FAKE_WS, need, nullptr), RKV_OK);
}

static void sizes_and_strings() {
  // the largest valid shapes (65535 slices at most): the workspace
  // arithmetic stays in range
  rkv_params p = P();
  p.num_layers = RKV_MAX_LAYERS;
  p.batch = 63;
  p.num_kv_heads = 8;
  p.capacity = RKV_MAX_CAPACITY;
  p.budget = RKV_MAX_CAPACITY - 128;
  const size_t n = rkv_workspace_bytes(&p);
  if (n < (size_t)RKV_MAX_LAYERS * 63 * 8 * RKV_MAX_CAPACITY * 12) {
    fprintf(stderr, "workspace of the largest shape: %zu\n", n);
    ++failures;
  }
  for (int s = -3; s < 12; ++s) {
    const char* str = rkv_status_string((rkv_status)s);
    if (!str || !*str) {
      fprintf(stderr, "status %d has no string\n", s);
      ++failures;
    }
  }
  EXPECT(rkv_last_hip_error(), 0);
}

int main() {
  bad_params();
  pointers_and_ranges();
  no_launch_paths();
  sizes_and_strings();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host layer: every call clean\n");
  return 0;
}
