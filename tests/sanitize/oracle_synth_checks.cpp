// Runs every entry point of the CPU oracle (oracle/rkv_oracle.h) and of the
// seeded input generator (synth/rkv_synth.c) on small inputs, normal cases
// and the degenerate ones (no-op below the trigger, N = B + 1, a window one
// short of the budget, zero and duplicate keys, negative threshold, empty
// decode, malformed keep lists), so that a build with AddressSanitizer and
// UndefinedBehaviorSanitizer sees every path. Exit status 0 when every call
// returned what its contract says; the sanitizers abort on any finding.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "rkv_oracle.h"

extern "C" {
uint64_t synth_stream_key(uint64_t seed, int64_t workload, int64_t tensor, int64_t layer, int64_t seq, int64_t head);
uint16_t synth_bf16_from_f32(float f);
void synth_fill_normal(uint64_t key, double mean, double sigma, int32_t dtype, void* out, int64_t n);
int32_t synth_slice_keys(uint64_t key, int32_t n, int32_t d, int32_t span_len, int32_t first_span, int32_t last_span,
                         int32_t n_copies, double noise_sigma, int32_t dtype, void* out, int32_t* copy_log);
void synth_mixture_means(uint64_t key, int32_t n_comp, int32_t d, double mean_sigma, double* means);
void synth_mixture_drift(uint64_t key, int32_t n_comp, int32_t d, double drift_sigma, double* means);
void synth_mixture_tokens(uint64_t key, int32_t n, int32_t d, int32_t n_comp, const double* means, int32_t dtype,
                          void* out);
int32_t synth_repeat_plan(uint64_t key, int32_t n_new, int32_t block_len, double p, int32_t pool_rows, int32_t* src);
void synth_repeat_apply(uint64_t key, int32_t n_new, int32_t d, int32_t block_len, const int32_t* src,
                        double noise_sigma, const void* windows, int32_t dtype, void* fresh);
void synth_fill_uniform_open(uint64_t key, float* out, int64_t n);
}

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static const int D = 128;

static size_t esize(int dtype) { return dtype == ORC_BF16 ? 2 : 4; }

// Keys of one slice with copied spans, in a buffer of exactly n rows.
static std::vector<unsigned char> slice_keys(uint64_t key, int n, int dtype, int copies) {
  std::vector<unsigned char> k((size_t)n * D * esize(dtype));
  std::vector<int32_t> log(2 * (copies > 0 ? copies : 1));
  const int span = 4, spans = n / span;
  synth_slice_keys(key, n, D, span, 1, spans > 1 ? spans - 1 : 1, copies, 0.05, dtype, k.data(), log.data());
  return k;
}

static std::vector<unsigned char> normal(uint64_t key, size_t count, int dtype) {
  std::vector<unsigned char> v(count * esize(dtype));
  synth_fill_normal(key, 0.0, 1.0, dtype, v.data(), (int64_t)count);
  return v;
}

// One slice with every output requested; returns the kept count.
static int run_slice(int n, int budget, int alpha, int group, double tau, int dtype, const void* keys,
                     const void* queries, const double* penalty) {
  orc_slice_params p = {n, D, group, alpha, budget, 2, 0.1, tau, 1e-6};
  std::vector<double> imp(n), rm(n), rbar(n), R(n), Z(n);
  std::vector<int32_t> cnt(n), amb(n), keep(n < budget ? n : budget);
  orc_slice_out o = {imp.data(), rm.data(), cnt.data(), rbar.data(), R.data(), Z.data(), amb.data(), keep.data()};
  const int kept = penalty ? orc_slice_penalized(&p, dtype, keys, queries, penalty, &o)
                           : orc_slice(&p, dtype, keys, queries, &o);
  CHECK(kept == (n < budget ? n : budget));
  for (int i = 1; i < kept; ++i) CHECK(keep[i - 1] < keep[i]);
  // the observation window is always kept
  if (kept == budget)
    for (int t = 0; t < alpha && t < n; ++t) CHECK(keep[kept - 1 - t] == n - 1 - t);
  return kept;
}

static void slices() {
  for (int dtype = ORC_BF16; dtype <= ORC_F32; ++dtype) {
    const int group = 2, alpha = 8;
    std::vector<unsigned char> q = normal(synth_stream_key(3, 1, 2, 0, 0, 0), (size_t)group * alpha * D, dtype);
    for (int n : {1, 20, 40, 41, 48, 97}) {
      std::vector<unsigned char> k = slice_keys(synth_stream_key(3, 1, 1, n, dtype, 0), n, dtype, n / 16);
      run_slice(n, 40, alpha, group, 0.5, dtype, k.data(), q.data(), nullptr);
      run_slice(n, 40, alpha, group, -0.3, dtype, k.data(), q.data(), nullptr);
      run_slice(n, 9, alpha, group, 0.5, dtype, k.data(), q.data(), nullptr);  // window one short of the budget
      std::vector<double> pen(n);
      for (int i = 0; i < n; ++i) pen[i] = (i % 5) * 0.01;
      run_slice(n, 40, alpha, group, 0.5, dtype, k.data(), q.data(), pen.data());
    }
    // zero keys and exact duplicates
    const int n = 50;
    std::vector<unsigned char> k = slice_keys(synth_stream_key(3, 1, 1, 999, dtype, 0), n, dtype, 0);
    memset(k.data(), 0, 3 * D * esize(dtype));
    memcpy(k.data() + 10 * D * esize(dtype), k.data() + 20 * D * esize(dtype), D * esize(dtype));
    run_slice(n, 40, alpha, group, 0.5, dtype, k.data(), q.data(), nullptr);
    // invalid parameters
    orc_slice_params bad = {n, D, group, alpha, alpha, 2, 0.1, 0.5, 0.0};
    orc_slice_out none = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    CHECK(orc_slice(&bad, dtype, k.data(), q.data(), &none) == -1);
    bad.budget = 40;
    bad.head_dim = 0;
    CHECK(orc_slice(&bad, dtype, k.data(), q.data(), &none) == -1);
  }
}

static void step(int dtype, double tau) {
  const int L = 2, B = 2, H = 2, G = 2, A = 8, budget = 40, buffer = 8, cap = 48;
  orc_step_params p = {L, B, H, G, D, cap, budget, buffer, A, 2, 0.1, tau};
  std::vector<std::vector<unsigned char>> K(L), V(L);
  std::vector<void*> kp(L), vp(L);
  for (int l = 0; l < L; ++l) {
    K[l] = normal(synth_stream_key(5, 2, 0, l, 0, 0), (size_t)B * H * cap * D, dtype);
    V[l] = normal(synth_stream_key(5, 2, 1, l, 0, 0), (size_t)B * H * cap * D, dtype);
    kp[l] = K[l].data();
    vp[l] = V[l].data();
  }
  std::vector<unsigned char> q = normal(synth_stream_key(5, 2, 2, 0, 0, 0), (size_t)L * B * H * G * A * D, dtype);
  std::vector<int32_t> keep((size_t)L * B * H * budget);
  int32_t seq_start[B] = {0, 11};  // the second sequence left-padded
  int32_t n_slots = cap - 1;
  CHECK(orc_evict_step(&p, dtype, kp.data(), vp.data(), q.data(), seq_start, &n_slots, keep.data()) == 0);
  CHECK(n_slots == cap - 1);
  n_slots = cap;
  CHECK(orc_evict_step(&p, dtype, kp.data(), vp.data(), q.data(), seq_start, &n_slots, keep.data()) == 1);
  CHECK(n_slots == budget);
  // sequence 0 keeps the budget; sequence 1 (cap - 11 valid tokens, below it) keeps all of them
  CHECK(seq_start[0] == 0 && seq_start[1] == budget - (cap - 11));
  orc_step_params bad = p;
  bad.capacity = budget;
  n_slots = cap;
  CHECK(orc_evict_step(&bad, dtype, kp.data(), vp.data(), q.data(), seq_start, &n_slots, nullptr) == -1);
}

static void holefill() {
  const int budget = 24, buffer = 8, n = budget + buffer, rb = D * 2;
  std::vector<unsigned char> k = slice_keys(synth_stream_key(7, 3, 0, 0, 0, 0), n, ORC_BF16, 2);
  std::vector<unsigned char> v = normal(synth_stream_key(7, 3, 1, 0, 0, 0), (size_t)n * D, ORC_BF16);
  std::vector<unsigned char> q = normal(synth_stream_key(7, 3, 2, 0, 0, 0), (size_t)2 * 8 * D, ORC_BF16);
  orc_slice_params p = {n, D, 2, 8, budget, 2, 0.1, 0.5, 0.0};
  std::vector<int32_t> kept(budget);
  orc_slice_out o = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, kept.data()};
  CHECK(orc_slice(&p, ORC_BF16, k.data(), q.data(), &o) == budget);
  std::vector<int32_t> order(budget);
  for (int i = 0; i < budget; ++i) order[i] = (i * 7 + 3) % budget;  // a permutation (7 is prime to 24)
  CHECK(orc_holefill_slice(k.data(), v.data(), rb, budget, n, kept.data(), order.data()) == 0);
  for (int i = 0; i < budget; ++i) order[i] = i;
  std::vector<int32_t> bad(kept);
  bad[0] = bad[1];  // not ascending
  CHECK(orc_holefill_slice(k.data(), v.data(), rb, budget, n, bad.data(), order.data()) == -1);
  order[1] = order[0];  // not a permutation
  CHECK(orc_holefill_slice(k.data(), v.data(), rb, budget, n, kept.data(), order.data()) == -1);
  std::vector<unsigned char> dst((size_t)budget * rb);
  orc_gather_rows(k.data(), kept.data(), budget, rb, dst.data());
}

static void decode() {
  for (int dtype = ORC_BF16; dtype <= ORC_F32; ++dtype)
    for (int n : {0, 1, 37}) {
      const int group = 4;
      std::vector<unsigned char> k = normal(synth_stream_key(9, 4, 0, n, 0, 0), (size_t)(n ? n : 1) * D, dtype);
      std::vector<unsigned char> v = normal(synth_stream_key(9, 4, 1, n, 0, 0), (size_t)(n ? n : 1) * D, dtype);
      std::vector<unsigned char> q = normal(synth_stream_key(9, 4, 2, n, 0, 0), (size_t)group * D, dtype);
      std::vector<double> out((size_t)group * D), w((size_t)group * (n ? n : 1));
      CHECK(orc_decode_attention(n, D, group, dtype, k.data(), v.data(), q.data(), out.data(), w.data()) == 0);
      CHECK(orc_decode_attention(n, D, group, dtype, k.data(), v.data(), q.data(), out.data(), nullptr) == 0);
    }
  double out[D];
  CHECK(orc_decode_attention(-1, D, 1, ORC_F32, nullptr, nullptr, nullptr, out, nullptr) == -1);
}

static void sentences() {
  for (int n_sent : {0, 1, 6}) {
    const int dim = 32;
    std::vector<float> vec((size_t)(n_sent ? n_sent : 1) * dim);
    synth_fill_normal(synth_stream_key(11, 5, 0, n_sent, 0, 0), 0.0, 1.0, ORC_F32, vec.data(),
                      (int64_t)n_sent * dim);
    if (n_sent > 2) {
      memset(vec.data() + dim, 0, dim * sizeof(float));  // a zero vector
      memcpy(vec.data() + 2 * dim, vec.data(), dim * sizeof(float));
    }
    std::vector<double> pen(n_sent ? n_sent : 1);
    orc_sentence_penalty(n_sent, dim, vec.data(), 0.5, pen.data());
  }
}

static void sampled() {
  const int n = 60;
  std::vector<float> s(n), u(n);
  synth_fill_uniform_open(synth_stream_key(13, 6, 0, 0, 0, 0), u.data(), n);
  synth_fill_normal(synth_stream_key(13, 6, 1, 0, 0, 0), 0.0, 1.0, ORC_F32, s.data(), n);
  std::vector<int32_t> keep(n);
  CHECK(orc_select_sampled(n, 24, 8, 30, 0.5, s.data(), u.data(), keep.data()) == 24);
  CHECK(orc_select_sampled(n, 24, 0, 0, 1.0, s.data(), u.data(), keep.data()) == 24);
  CHECK(orc_select_sampled(n, 24, 23, 1000, 1e-3, s.data(), u.data(), keep.data()) == 24);
  CHECK(orc_select_sampled(10, 24, 8, 30, 0.5, s.data(), u.data(), keep.data()) == 10);
  CHECK(orc_select_sampled(n, 24, 8, 30, 0.0, s.data(), u.data(), keep.data()) == -1);
  CHECK(orc_select_sampled(n, 24, 25, 30, 1.0, s.data(), u.data(), keep.data()) == -1);
}

static void synth_rest() {
  const int comps = 3, n_new = 40, blk = 8;
  std::vector<double> means((size_t)comps * D);
  synth_mixture_means(synth_stream_key(17, 7, 0, 0, 0, 0), comps, D, 2.0, means.data());
  synth_mixture_drift(synth_stream_key(17, 7, 1, 0, 0, 0), comps, D, 0.1, means.data());
  std::vector<uint16_t> fresh((size_t)n_new * D);
  synth_mixture_tokens(synth_stream_key(17, 7, 2, 0, 0, 0), n_new, D, comps, means.data(), ORC_BF16, fresh.data());
  std::vector<int32_t> src(n_new / blk);
  const int rep = synth_repeat_plan(synth_stream_key(17, 7, 3, 0, 0, 0), n_new, blk, 0.5, 30, src.data());
  std::vector<uint16_t> windows((size_t)(rep ? rep : 1) * blk * D, synth_bf16_from_f32(0.25f));
  synth_repeat_apply(synth_stream_key(17, 7, 4, 0, 0, 0), n_new, D, blk, src.data(), 0.05, windows.data(), ORC_BF16,
                     fresh.data());
  CHECK(synth_repeat_plan(synth_stream_key(17, 7, 5, 0, 0, 0), n_new, blk, 1.0, blk - 1, src.data()) == 0);
}

int main() {
  slices();
  for (int dtype = ORC_BF16; dtype <= ORC_F32; ++dtype) {
    step(dtype, 0.5);
    step(dtype, -0.3);
  }
  holefill();
  decode();
  sentences();
  sampled();
  synth_rest();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle and generator: every call clean\n");
  return 0;
}
