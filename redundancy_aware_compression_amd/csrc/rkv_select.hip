// K4 — per-head selection: redundancy softmax, score combination and an
// exact top-k by LDS radix select.
//
// R-KV notes page (yoonschallenge.tistory.com/1236): opening notes (keep the
// newest 8 tokens, keep the top-scoring rest up to the budget, drop the
// others); summary table row "final selection criterion" (importance raises
// the score, redundancy lowers it, lambda = 0.1; the formula itself is not
// printed — Z = lambda*I - (1-lambda)*R is the stated reading); Q&A part 2,
// cause 3 (redundancy softmax, combination, top-k selection).
//
// One work-group per (layer, sequence, KV head): R = softmax of the
// redundancy over the candidates, Z per candidate, Z mapped to an
// order-preserving uint32 key (+0 and -0 equal), four 8-bit radix passes over
// LDS histograms find the k-th largest key exactly, equal keys are resolved
// towards the later slot with a suffix count, and a block prefix sum writes
// the kept slots in ascending order. Deterministic: no float atomics, every
// reduction has a fixed order.
#include "rkv_select.hpp"

namespace rkv {

// FROM_COUNTS: redundancy = counts < beta ? 0 : rowmean (the eviction step);
// otherwise read the given redundancy array (the standalone select call).
// PEN: SkipKV's sentence deduction (SkipKV notes page, summary table row
// "final eviction score"): Z of a candidate loses the penalty of its slot's
// sentence, sent_pen[b][sent_id[slot]] (ids outside [0, s_max): none).
template <bool FROM_COUNTS, bool PEN>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(Geom g, const float* __restrict__ importance,
                                                                const float* __restrict__ redundancy,
                                                                const int32_t* __restrict__ counts,
                                                                const float* __restrict__ rowmean,
                                                                const int32_t* __restrict__ seq_start,
                                                                int32_t* __restrict__ keep, float* __restrict__ z_out,
                                                                float* __restrict__ r_out,
                                                                const float* __restrict__ sent_pen,
                                                                const int32_t* __restrict__ sent_id, int s_max) {
  extern __shared__ uint32_t keys[];  // dynamic: n_slots entries (select_lds_bytes)
  __shared__ __align__(16) SelectLds sm;
  const int slice = blockIdx.x;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  select_slice<FROM_COUNTS, PEN>(g, slice, b, s0, N, importance, redundancy, counts, rowmean, keep, z_out, r_out,
                                 sent_pen, sent_id, s_max, keys, sm);
}

// ---------------------------------------------------------------------------
// Sampled selection (ForesightKV page, technical summary: when the cache
// reaches budget + L, the newest L tokens stay and the rest is compressed to
// budget - L by a Top-K followed by multinomial sampling on the scores of a
// learned scoring model; the scores are the caller's). Per slice, among the
// candidates (every valid token but the newest keep_newest): the top_k by
// score (equal scores: the later slot), then budget - keep_newest of those
// drawn without replacement with probabilities proportional to
// exp(score / temperature). The draw is the Gumbel-top-k form of that
// sampling: the largest score / temperature - log(-log u) among the top_k,
// u the caller's uniform in (0, 1) for the slot (the same law as drawing one
// token at a time, each with probability proportional to exp(score / T)
// among those left).
__global__ __launch_bounds__(kSelectThreads) void select_sampled_kernel(Geom g, const float* __restrict__ scores,
                                                                        const float* __restrict__ uniforms,
                                                                        const int32_t* __restrict__ seq_start,
                                                                        int keep_newest, int top_k, float inv_temp,
                                                                        int32_t* __restrict__ keep) {
  extern __shared__ uint32_t keys[];  // dynamic: n_slots entries (select_lds_bytes)
  __shared__ __align__(16) int hist[2 * kHistInts];
  __shared__ int iscr[16];
  __shared__ int sel[2];

  const int slice = blockIdx.x;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  const int tid = threadIdx.x, nt = blockDim.x;
  int32_t* krow = keep + (size_t)slice * g.budget;
  const int B = g.budget;
  if (N <= B) {  // keep every valid token, right-aligned
    for (int j = tid; j < B; j += nt) krow[j] = j >= B - N ? j + (g.n_slots - B) : -1;
    return;
  }
  const int nc = N - keep_newest, kk = B - keep_newest;
  const int K = min(max(top_k, kk), nc);
  const size_t base = (size_t)slice * g.n_slots + s0;
  constexpr int E = 8;  // loads per thread issued together
  for (int i0 = tid; i0 < nc; i0 += E * nt) {
    float sc[E];
#pragma unroll
    for (int u = 0; u < E; ++u) sc[u] = scores[base + min(i0 + u * nt, nc - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < E; ++u)
      if (i0 + u * nt < nc) keys[i0 + u * nt] = order_key(sc[u]);
  }
  __syncthreads();
  // each thread owns a contiguous range of the valid tokens
  const int seg = (N + nt - 1) / nt;
  const int lo = tid * seg, hi = min(N, lo + seg);
  // 1. the top K by score; survivors get their Gumbel key, the rest key 0
  //    (below every float's key)
  {
    uint32_t T;
    int need;
    radix_kth(keys, nc, K, hist, sel, T, need);
    int eq_here = 0;
    for (int i = lo; i < hi && i < nc; ++i) eq_here += keys[i] == T;
    int eq_total;
    const int eq_before = block_exclusive_scan(eq_here, iscr, &eq_total);
    int ea = eq_total - eq_before - eq_here;
    // the thread's candidates from the newest down, E at a time (their
    // uniforms and scores loaded together)
    for (int c = min(hi, nc) - 1; c >= lo; c -= E) {
      float uv[E], sv[E];
#pragma unroll
      for (int u = 0; u < E; ++u) {
        const int i = max(c - u, lo);
        uv[u] = uniforms[base + i];
        sv[u] = scores[base + i];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < E; ++u) {
        const int i = c - u;
        if (i >= lo) {
          const uint32_t key = keys[i];
          const bool take = key > T || (key == T && ea < need);
          if (key == T) ++ea;
          keys[i] = take ? order_key(sv[u] * inv_temp - logf(-logf(uv[u]))) : 0u;
        }
      }
    }
    __syncthreads();
  }
  // 2. the top kk of the Gumbel keys, then the kept slots in ascending order
  uint32_t T;
  int need;
  radix_kth(keys, nc, kk, hist, sel, T, need);
  int eq_here = 0;
  for (int i = lo; i < hi && i < nc; ++i) eq_here += keys[i] == T;
  int eq_total;
  const int eq_before = block_exclusive_scan(eq_here, iscr, &eq_total);
  const int eq_after = eq_total - eq_before - eq_here;
  int kept_here = 0;
  {
    int ea = eq_after;
    for (int i = hi - 1; i >= lo; --i) {
      bool take = true;  // the newest keep_newest tokens
      if (i < nc) {
        const uint32_t key = keys[i];
        take = key > T || (key == T && ea < need);
        if (key == T) ++ea;
      }
      kept_here += take;
    }
  }
  int kept_total;
  const int out = block_exclusive_scan(kept_here, iscr, &kept_total);
  {
    int ea = eq_after;
    int pos = out + kept_here;
    for (int i = hi - 1; i >= lo; --i) {
      bool take = true;
      if (i < nc) {
        const uint32_t key = keys[i];
        take = key > T || (key == T && ea < need);
        if (key == T) ++ea;
      }
      if (take && --pos < B) krow[pos] = s0 + i;
    }
  }
}

// The keys of a slice's candidates live in dynamic LDS sized for n_slots, so
// short slices leave room for more work-groups per compute unit.
static size_t select_lds_bytes(const Geom& g) { return (size_t)(g.n_slots > 0 ? g.n_slots : 1) * 4; }

// Allows `kernel` dynamic LDS beyond the default 64 KB when it needs it.
static int allow_lds(const void* kernel, size_t lds) {
  if (lds <= 48 * 1024) return 0;
  return (int)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

int launch_select_sampled(const Geom& g, const float* scores, const float* uniforms, const int32_t* seq_start,
                          int keep_newest, int top_k, float temperature, int32_t* keep, void* stream) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  const size_t lds = select_lds_bytes(g);
  if (const int e = allow_lds((const void*)select_sampled_kernel, lds)) return e;
  RKV_LAUNCH(select_sampled_kernel, dim3(slices), dim3(kSelectThreads), lds, (hipStream_t)stream, g, scores,
             uniforms, seq_start, keep_newest, top_k, 1.f / temperature, keep);
  return 0;
}

int launch_select(const Geom& g, const float* importance, const float* redundancy, const int32_t* counts,
                  const float* rowmean, const int32_t* seq_start, int32_t* keep, float* z_out, float* r_out,
                  void* stream, const float* sent_pen, const int32_t* sent_id, int s_max) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(slices), block(kSelectThreads);
  const size_t lds = select_lds_bytes(g);
#define RKV_SELECT(FC, PEN)                                                                              \
  do {                                                                                                   \
    if (const int e = allow_lds((const void*)select_kernel<FC, PEN>, lds)) return e;                     \
    RKV_LAUNCH((select_kernel<FC, PEN>), grid, block, lds, s, g, importance, redundancy, counts, rowmean, \
               seq_start, keep, z_out, r_out, sent_pen, sent_id, s_max);                                 \
  } while (0)
  if (counts && sent_pen)
    RKV_SELECT(true, true);
  else if (counts)
    RKV_SELECT(true, false);
  else
    RKV_SELECT(false, false);
#undef RKV_SELECT
  return 0;
}

}  // namespace rkv
