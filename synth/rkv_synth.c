/*
 * Seeded synthetic inputs for the R-KV eviction step: key, value and
 * observation-query tensors with repeated-span structure.
 *
 * This module is shared by the CPU oracle side and the HIP side of the tests
 * and the benchmark. It holds no arithmetic of the eviction method itself:
 * it only draws numbers, rounds them to the storage type and copies spans.
 *
 * Generators, each written from its published definition:
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014), used both as the stream generator and, via
 *     its output mix, to derive one independent stream per
 *     (workload, seed, tensor, layer, sequence, head) tuple.
 *   - Box-Muller transform (1958) for normal deviates, evaluated in double.
 *   - IEEE-754 binary32 -> bfloat16 round-to-nearest-even.
 *
 * Every function writes only caller-owned memory and is reentrant.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_BF16 0
#define SYNTH_F32 1

typedef struct {
  uint64_t state;
  int have_spare;
  double spare;
} synth_stream;

static uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t sm64_next(synth_stream* s) {
  s->state += 0x9E3779B97F4A7C15ULL;
  return sm64_mix(s->state);
}

/* Uniform double in [0, 1) from the top 53 bits. */
static double unif01(synth_stream* s) {
  return (double)(sm64_next(s) >> 11) * (1.0 / 9007199254740992.0);
}

/* Uniform integer in [0, m), m >= 1. */
static int64_t unif_int(synth_stream* s, int64_t m) {
  int64_t v = (int64_t)(unif01(s) * (double)m);
  return v >= m ? m - 1 : v;
}

static double normal01(synth_stream* s) {
  if (s->have_spare) {
    s->have_spare = 0;
    return s->spare;
  }
  /* u1 in (0, 1] so that log(u1) is finite. */
  double u1 = (double)((sm64_next(s) >> 11) + 1) * (1.0 / 9007199254740992.0);
  double u2 = unif01(s);
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  s->spare = r * sin(th);
  s->have_spare = 1;
  return r * cos(th);
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return 0x7FC0; /* NaN */
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

static float bf16_to_f32(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

static void store_val(void* out, int32_t dtype, int64_t idx, double v) {
  float f = (float)v;
  if (dtype == SYNTH_BF16)
    ((uint16_t*)out)[idx] = f32_to_bf16_rne(f);
  else
    ((float*)out)[idx] = f;
}

static double load_val(const void* in, int32_t dtype, int64_t idx) {
  if (dtype == SYNTH_BF16) return (double)bf16_to_f32(((const uint16_t*)in)[idx]);
  return (double)((const float*)in)[idx];
}

/* Derives the stream key of one (workload, seed, tensor, layer, sequence, head). */
uint64_t synth_stream_key(uint64_t seed, int64_t workload, int64_t tensor, int64_t layer,
                          int64_t seq, int64_t head) {
  int64_t f[5] = {workload, tensor, layer, seq, head};
  uint64_t k = sm64_mix(seed + 0x9E3779B97F4A7C15ULL);
  for (int i = 0; i < 5; ++i) k = sm64_mix(k ^ ((uint64_t)f[i] + 0x9E3779B97F4A7C15ULL * (uint64_t)(i + 2)));
  return k;
}

uint16_t synth_bf16_from_f32(float f) { return f32_to_bf16_rne(f); }

/* out[i] = mean + sigma * N(0,1), rounded to dtype, for i < n. */
void synth_fill_normal(uint64_t key, double mean, double sigma, int32_t dtype, void* out, int64_t n) {
  synth_stream s = {key, 0, 0.0};
  for (int64_t i = 0; i < n; ++i) store_val(out, dtype, i, mean + sigma * normal01(&s));
}

/* Draws `count` distinct integers from [lo, hi] (partial Fisher-Yates) and
 * returns them sorted ascending in out[0..count). Returns the count drawn. */
static int32_t draw_distinct_sorted(synth_stream* s, int32_t lo, int32_t hi, int32_t count, int32_t* out) {
  int32_t m = hi - lo + 1;
  if (m <= 0) return 0;
  if (count > m) count = m;
  int32_t* pool = (int32_t*)malloc(sizeof(int32_t) * (size_t)m);
  if (!pool) return 0;
  for (int32_t i = 0; i < m; ++i) pool[i] = lo + i;
  for (int32_t i = 0; i < count; ++i) {
    int32_t j = i + (int32_t)unif_int(s, m - i);
    int32_t t = pool[i];
    pool[i] = pool[j];
    pool[j] = t;
  }
  for (int32_t i = 0; i < count; ++i) out[i] = pool[i];
  free(pool);
  /* insertion sort: counts are small */
  for (int32_t i = 1; i < count; ++i) {
    int32_t v = out[i], j = i - 1;
    while (j >= 0 && out[j] > v) {
      out[j + 1] = out[j];
      --j;
    }
    out[j + 1] = v;
  }
  return count;
}

/*
 * Keys of one slice with repeated spans: n rows of d values, row-major.
 * Every value starts as N(0,1). Then `n_copies` distinct destination spans
 * (span index in [first_span, last_span], span s covering rows
 * [s*span_len, (s+1)*span_len)) are chosen uniformly; in ascending order each
 * one is overwritten by a copy of a uniformly placed earlier window
 * [src, src+span_len) with src in [0, s*span_len - span_len], plus
 * N(0, noise_sigma^2) per value. A destination row beyond n is skipped.
 * copy_log (nullable, 2*n_copies ints) receives (dst_row, src_row) pairs.
 * Returns the number of copies made.
 */
int32_t synth_slice_keys(uint64_t key, int32_t n, int32_t d, int32_t span_len, int32_t first_span,
                         int32_t last_span, int32_t n_copies, double noise_sigma, int32_t dtype, void* out,
                         int32_t* copy_log) {
  synth_stream s = {key, 0, 0.0};
  for (int64_t i = 0; i < (int64_t)n * d; ++i) store_val(out, dtype, i, normal01(&s));
  if (n_copies <= 0 || span_len <= 0) return 0;
  int32_t* spans = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_copies);
  if (!spans) return 0;
  int32_t got = draw_distinct_sorted(&s, first_span, last_span, n_copies, spans);
  for (int32_t c = 0; c < got; ++c) {
    int64_t dst = (int64_t)spans[c] * span_len;
    int64_t src_hi = dst - span_len; /* inclusive upper bound of the source start */
    int64_t src = src_hi > 0 ? unif_int(&s, src_hi + 1) : 0;
    if (copy_log) {
      copy_log[2 * c] = (int32_t)dst;
      copy_log[2 * c + 1] = (int32_t)src;
    }
    for (int64_t r = 0; r < span_len; ++r) {
      if (dst + r >= n) break;
      for (int64_t e = 0; e < d; ++e) {
        double v = load_val(out, dtype, (src + r) * d + e) + noise_sigma * normal01(&s);
        store_val(out, dtype, (dst + r) * d + e, v);
      }
    }
  }
  free(spans);
  return got;
}

/*
 * Gaussian-mixture tokens for the long-generation sweep.
 * synth_mixture_means: means[c*d + e] = N(0, mean_sigma^2), c < n_comp.
 * synth_mixture_drift: means += N(0, drift_sigma^2) elementwise.
 * synth_mixture_tokens: for each of n rows, a component c uniform in
 *   [0, n_comp) and value means[c] + N(0, 1), rounded to dtype.
 */
void synth_mixture_means(uint64_t key, int32_t n_comp, int32_t d, double mean_sigma, double* means) {
  synth_stream s = {key, 0, 0.0};
  for (int64_t i = 0; i < (int64_t)n_comp * d; ++i) means[i] = mean_sigma * normal01(&s);
}

void synth_mixture_drift(uint64_t key, int32_t n_comp, int32_t d, double drift_sigma, double* means) {
  synth_stream s = {key, 0, 0.0};
  for (int64_t i = 0; i < (int64_t)n_comp * d; ++i) means[i] += drift_sigma * normal01(&s);
}

void synth_mixture_tokens(uint64_t key, int32_t n, int32_t d, int32_t n_comp, const double* means,
                          int32_t dtype, void* out) {
  synth_stream s = {key, 0, 0.0};
  for (int64_t r = 0; r < n; ++r) {
    int64_t c = unif_int(&s, n_comp);
    for (int64_t e = 0; e < d; ++e) store_val(out, dtype, r * d + e, means[c * d + e] + normal01(&s));
  }
}

/*
 * Repeat injection for the long-generation sweep, in two steps so that the
 * copied windows can be fetched from wherever the retained cache lives.
 * synth_repeat_plan: the n_new new rows are taken in blocks of block_len;
 *   for block i a uniform u and a window start src uniform in
 *   [0, pool_rows - block_len] are drawn, and the block is replaced iff
 *   u < p (src[i] = start) or kept (src[i] = -1). Returns the number of
 *   replaced blocks (none when pool_rows < block_len).
 * synth_repeat_apply: the w-th replaced block (in block order) becomes
 *   windows[w] + N(0, noise_sigma^2) elementwise, rounded to dtype; windows
 *   holds the replaced blocks' source rows, [replaced][block_len][d].
 */
int32_t synth_repeat_plan(uint64_t key, int32_t n_new, int32_t block_len, double p, int32_t pool_rows,
                          int32_t* src) {
  synth_stream s = {key, 0, 0.0};
  int32_t replaced = 0;
  for (int32_t i = 0; (int64_t)(i + 1) * block_len <= n_new; ++i) {
    const double u = unif01(&s);
    const int64_t start = pool_rows >= block_len ? unif_int(&s, (int64_t)pool_rows - block_len + 1) : 0;
    src[i] = (pool_rows >= block_len && u < p) ? (int32_t)start : -1;
    replaced += src[i] >= 0;
  }
  return replaced;
}

void synth_repeat_apply(uint64_t key, int32_t n_new, int32_t d, int32_t block_len, const int32_t* src,
                        double noise_sigma, const void* windows, int32_t dtype, void* fresh) {
  synth_stream s = {key, 0, 0.0};
  int64_t w = 0;
  for (int32_t i = 0; (int64_t)(i + 1) * block_len <= n_new; ++i) {
    if (src[i] < 0) continue;
    for (int64_t r = 0; r < block_len; ++r)
      for (int64_t e = 0; e < d; ++e) {
        const double v = load_val(windows, dtype, (w * block_len + r) * d + e) + noise_sigma * normal01(&s);
        store_val(fresh, dtype, ((int64_t)i * block_len + r) * d + e, v);
      }
    ++w;
  }
}

/* out[i] = a float32 uniform strictly inside (0, 1): (24 random bits + 1/2)
 * / 2^24, exact in float32, for i < n. */
void synth_fill_uniform_open(uint64_t key, float* out, int64_t n) {
  synth_stream s = {key, 0, 0.0};
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(((double)(sm64_next(&s) >> 40) + 0.5) * (1.0 / 16777216.0));
}
