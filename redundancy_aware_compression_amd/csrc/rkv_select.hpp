// Selection of one slice (R-KV's redundancy softmax, score combination and
// exact top-k), shared by the selection kernel and the fused eviction-step
// kernel: the work-group of the slice calls select_slice with every thread.
//
// R-KV notes page (yoonschallenge.tistory.com/1236): opening notes (keep the
// newest 8 tokens, keep the top-scoring rest up to the budget, drop the
// others); summary table row "final selection criterion" (importance raises
// the score, redundancy lowers it, lambda = 0.1; the formula itself is not
// printed — Z = lambda*I - (1-lambda)*R is the stated reading); Q&A part 2,
// cause 3 (redundancy softmax, combination, top-k selection).
#pragma once

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

// LDS of one slice's selection besides its keys (n_slots words).
struct SelectLds {
  int hist[2 * kHistInts];
  float fscr[16];
  int iscr[16];
  int sel[2];
};

// FROM_COUNTS: redundancy = counts < beta ? 0 : rowmean (the eviction step);
// otherwise read the given redundancy array (the standalone select call).
// PEN: SkipKV's sentence deduction (SkipKV notes page, summary table row
// "final eviction score"): Z of a candidate loses the penalty of its slot's
// sentence, sent_pen[b][sent_id[slot]] (ids outside [0, s_max): none).
template <bool FROM_COUNTS, bool PEN>
__device__ inline void select_slice(const Geom& g, int slice, int b, int s0, int N, const float* __restrict__ importance,
                                    const float* __restrict__ redundancy, const int32_t* __restrict__ counts,
                                    const float* __restrict__ rowmean, int32_t* __restrict__ keep,
                                    float* __restrict__ z_out, float* __restrict__ r_out,
                                    const float* __restrict__ sent_pen, const int32_t* __restrict__ sent_id, int s_max,
                                    uint32_t* keys, SelectLds& sm) {
  int* hist = sm.hist;
  float* fscr = sm.fscr;
  int* iscr = sm.iscr;
  int* sel = sm.sel;
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

}  // namespace rkv
