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
#include "rkv_device.hpp"

namespace rkv {

constexpr int kSelectThreads = 512;

__device__ inline uint32_t order_key(float z) {
  uint32_t u = __float_as_uint(z);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact k-th largest of keys[0 .. n) (1 <= k <= n) by four 8-bit radix
// passes over LDS histograms: T is that key and `need` the number of keys
// equal to T among the top k. Every thread of the work-group takes part and
// receives both. hist holds two histograms of 256 bins (kHistInts ints each):
// while one pass's digit is found, the other is cleared for the next pass, so
// each pass needs two barriers. Each bin has kHistCopies adjacent counters and
// a thread adds into copy (tid % kHistCopies): the keys of a slice share their
// top bits (sign and exponent), so the first passes put nearly every key in a
// few bins, and same-address LDS atomics serialise. sel[0], sel[1]: the pass's
// digit and the keys above it. Every read of keys is done when this returns.
constexpr int kHistCopies = 4;
constexpr int kHistInts = 256 * kHistCopies;
__device__ inline void radix_kth(const uint32_t* keys, int n, int k, int* hist, int* sel, uint32_t& T, int& need) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint32_t prefix = 0;
  need = k;
  for (int d = tid; d < kHistInts; d += nt) hist[d] = 0;
  __syncthreads();
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    int* h = hist + (pass & 1) * kHistInts;
    int* hn = hist + ((pass + 1) & 1) * kHistInts;
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < n; i += nt) {
      const uint32_t key = keys[i];
      if ((key & hi_mask) == prefix) atomicAdd(&h[kHistCopies * ((key >> shift) & 255u) + (tid % kHistCopies)], 1);
    }
    __syncthreads();  // this pass's histogram is complete
    for (int d = tid; d < kHistInts; d += nt) hn[d] = 0;  // the next pass's, last read in the previous pass
    if (tid < 64) {
      // lane l owns digits 4l..4l+3; suffix sums from the top digit down
      static_assert(kHistCopies == 4, "one int4 per bin");
      const int4* h4 = (const int4*)h + 4 * tid;
      const int4 q0 = h4[0], q1 = h4[1], q2 = h4[2], q3 = h4[3];
      const int c0 = q0.x + q0.y + q0.z + q0.w, c1 = q1.x + q1.y + q1.z + q1.w, c2 = q2.x + q2.y + q2.z + q2.w,
                c3 = q3.x + q3.y + q3.z + q3.w;
      const int own = c0 + c1 + c2 + c3;
      const int pre = wave_prefix_sum(own);                       // lanes <= tid
      const int above_lane = __builtin_amdgcn_readlane(pre, 63) - pre;  // keys in digits above 4*tid+3
      // the digit d with above(d) < need <= above(d) + h[d] lies in exactly one lane
      int a3 = above_lane, a2 = a3 + c3, a1 = a2 + c2, a0 = a1 + c1;
      int d = -1, ab = 0;
      if (a3 < need && need <= a3 + c3) { d = 4 * tid + 3; ab = a3; }
      else if (a2 < need && need <= a2 + c2) { d = 4 * tid + 2; ab = a2; }
      else if (a1 < need && need <= a1 + c1) { d = 4 * tid + 1; ab = a1; }
      else if (a0 < need && need <= a0 + c0) { d = 4 * tid; ab = a0; }
      if (d >= 0) {
        sel[0] = d;
        sel[1] = ab;
      }
    }
    __syncthreads();  // the digit is chosen and the next histogram cleared
    need -= sel[1];
    prefix |= (uint32_t)sel[0] << shift;
  }
  T = prefix;
}

// Merges the softmax partials (m2, s2) into (m1, s1): s is a sum of exp(x - m).
__device__ inline void merge_softmax(float& m1, float& s1, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m1 == -INFINITY) {
    m1 = m2;
    s1 = s2;
    return;
  }
  const float m = fmaxf(m1, m2);
  s1 = s1 * __expf(m1 - m) + s2 * __expf(m2 - m);
  m1 = m;
}

// The merge over the 64 lanes of a wave, every lane receiving it: partners in
// DPP steps (lanes 1 and 2 apart in a quad, then the mirrored quad of each 8,
// the mirrored 8 of each row) and the half swaps for rows and halves. The
// merge is commutative, so both partners of a step hold the same result. The
// exec mask must be full.
template <int CTRL>
__device__ inline float dpp_partner(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}
__device__ inline void wave_merge_softmax(float& m, float& s) {
  merge_softmax(m, s, dpp_partner<0xB1>(m), dpp_partner<0xB1>(s));    // quad_perm [1, 0, 3, 2]
  merge_softmax(m, s, dpp_partner<0x4E>(m), dpp_partner<0x4E>(s));    // quad_perm [2, 3, 0, 1]
  merge_softmax(m, s, dpp_partner<0x141>(m), dpp_partner<0x141>(s));  // row_half_mirror
  merge_softmax(m, s, dpp_partner<0x140>(m), dpp_partner<0x140>(s));  // row_mirror
  merge_softmax(m, s, lane_xor16(m), lane_xor16(s));
  merge_softmax(m, s, lane_xor32(m), lane_xor32(s));
}

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
  __shared__ __align__(16) int hist[2 * kHistInts];
  __shared__ float fscr[16];
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
  const int nc = N - g.alpha, kk = B - g.alpha;
  const size_t base = (size_t)slice * g.n_slots + s0;
  float* fk = (float*)keys;

  // ---- redundancy softmax over the candidates: one pass keeps each thread's
  // running max and sum of exp, then the work-group merges them
  float mx = -INFINITY, sum = 0.f;
  constexpr int E = 8;  // elements per thread whose loads go out together
  for (int i0 = tid; i0 < nc; i0 += E * nt) {
    float rv[E];
    int cv[E];
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int i = min(i0 + u * nt, nc - 1);  // in range; the extra elements are not used
      if (FROM_COUNTS) {
        cv[u] = counts[base + i];
        rv[u] = rowmean[base + i];
      } else {
        rv[u] = redundancy[base + i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int i = i0 + u * nt;
      if (i < nc) {
        const float r = FROM_COUNTS ? (cv[u] < g.beta ? 0.f : rv[u]) : rv[u];
        fk[i] = r;
        if (r > mx) {
          sum = (mx == -INFINITY ? 0.f : sum * __expf(mx - r)) + 1.f;
          mx = r;
        } else {
          sum += __expf(r - mx);
        }
      }
    }
  }
  wave_merge_softmax(mx, sum);
  if ((tid & 63) == 0) {
    fscr[tid >> 6] = mx;
    fscr[8 + (tid >> 6)] = sum;
  }
  __syncthreads();
  mx = fscr[0];
  sum = fscr[8];
  for (int w = 1; w < nt / 64; ++w) merge_softmax(mx, sum, fscr[w], fscr[8 + w]);
  const float inv = 1.f / sum;
  for (int i0 = tid; i0 < nc; i0 += E * nt) {
    float iv[E];
    int sv[E];
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int i = min(i0 + u * nt, nc - 1);
      iv[u] = importance[base + i];
      if (PEN) sv[u] = sent_id[(size_t)slice * g.capacity + s0 + i];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int i = i0 + u * nt;
      if (i < nc) {
        const float R = __expf(fk[i] - mx) * inv;
        float Z = g.lambda * iv[u] - (1.f - g.lambda) * R;
        if (PEN) {
          const int sid = sv[u];
          Z -= (sid >= 0 && sid < s_max) ? sent_pen[(size_t)b * s_max + sid] : 0.f;
        }
        keys[i] = order_key(Z);
        if (z_out) z_out[base + i] = Z;
        if (r_out) r_out[base + i] = R;
      }
    }
  }
  __syncthreads();

  // ---- radix select: exact k-th largest key T, and how many keys equal to T to take
  uint32_t T;
  int need;
  radix_kth(keys, nc, kk, hist, sel, T, need);

  // ---- keys equal to T: keep the `need` latest ones. Each thread owns a
  // contiguous range of candidates; a suffix count over threads gives every
  // equal key the number of equal keys after it.
  const int seg = (N + nt - 1) / nt;
  const int lo = tid * seg, hi = min(N, lo + seg);
  int eq_here = 0;
  for (int i = lo; i < hi && i < nc; ++i) eq_here += keys[i] == T;
  int eq_total;
  const int eq_before = block_exclusive_scan(eq_here, iscr, &eq_total);
  int eq_after = eq_total - eq_before - eq_here;  // equal keys in later threads' ranges

  // ---- flags and their prefix sum give the output position of each kept slot
  int kept_here = 0;
  {
    int ea = eq_after;
    for (int i = hi - 1; i >= lo; --i) {
      bool take;
      if (i >= nc) {
        take = true;  // observation window
      } else {
        const uint32_t key = keys[i];
        take = key > T || (key == T && ea < need);
        if (key == T) ++ea;
      }
      kept_here += take;
    }
  }
  int kept_total;
  int out = block_exclusive_scan(kept_here, iscr, &kept_total);
  {
    int ea = eq_after;
    // walk backwards to reuse the suffix count, writing positions from the end of the range
    int pos = out + kept_here;
    for (int i = hi - 1; i >= lo; --i) {
      bool take;
      if (i >= nc) {
        take = true;
      } else {
        const uint32_t key = keys[i];
        take = key > T || (key == T && ea < need);
        if (key == T) ++ea;
      }
      if (take && --pos < B) krow[pos] = s0 + i;  // pos < B always; the guard only bounds the write
    }
  }
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
