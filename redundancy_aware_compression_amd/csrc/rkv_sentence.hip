// Sentence-level redundancy (SkipKV notes page, yoonschallenge.tistory.com/
// 1230, summary table rows "sentence-level KV storage skipping", "final
// eviction score" and "cache range monitoring"): a sentence is represented by
// the mean of its tokens' last-layer hidden states (the caller's vectors);
// when a later sentence's cosine with an earlier one exceeds a threshold the
// earlier one is redundant, and its tokens lose that similarity on the
// eviction score, so they go before ordinary tokens. Each cached slot carries
// its token's sentence id, a sidecar that moves with the slot's K/V rows so
// that sentence scores keep landing on the right cache entries after evictions.
#include "rkv_device.hpp"

namespace rkv {

constexpr int kSentThreads = 256;
constexpr int kSentBatch = 4;
constexpr int kSentChunk = 4;  // float4 per lane per sentence in one round of loads

// One work-group per (sentence i, sequence b): penalty[b][i] = the largest
// cosine of sentence i with a later sentence j < n_sent[b] when it exceeds
// tau_s, else 0 (a zero vector is similar to nothing). fp32 dot products over
// dim (a multiple of 4, at most kSentMaxDim); sentence i's vector is staged in
// LDS and the waves take the later sentences in batches.
template <int NT>
__global__ __launch_bounds__(NT) void sentence_penalty_kernel(const float* __restrict__ vectors,
                                                                        const int32_t* __restrict__ n_sent,
                                                                        int s_max, int dim, float tau_s,
                                                                        float* __restrict__ penalty) {
  extern __shared__ __align__(16) float hv[];
  __shared__ float red[NT / 64];
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int n = n_sent[b];
  n = n < 0 ? 0 : (n > s_max ? s_max : n);
  float* out = penalty + (size_t)b * s_max + i;
  if (i >= n) {
    if (tid == 0) *out = 0.f;
    return;
  }
  const float4* vi = (const float4*)(vectors + ((size_t)b * s_max + i) * dim);
  float ss = 0.f;
  for (int d = tid; d < dim / 4; d += NT) {
    const float4 x = vi[d];
    ((float4*)hv)[d] = x;
    ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
  }
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float ni = 0.f;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) ni += red[k];
  ni = sqrtf(ni);
  float best = -INFINITY;  // the wave's largest cosine above tau_s
  // Each wave takes kSentBatch later sentences at a time; their loads are
  // independent, so a batch costs about one memory round trip. Indexes past
  // the last sentence re-read sentence n - 1 and are discarded.
  for (int j0 = i + 1 + w * kSentBatch; j0 < n; j0 += NT / 64 * kSentBatch) {
    float dot[kSentBatch], sj[kSentBatch];
    const float4* vj[kSentBatch];
#pragma unroll
    for (int u = 0; u < kSentBatch; ++u) {
      dot[u] = 0.f;
      sj[u] = 0.f;
      vj[u] = (const float4*)(vectors + ((size_t)b * s_max + min(j0 + u, n - 1)) * dim);
    }
    for (int d0 = 0; d0 < dim / 4; d0 += 64 * kSentChunk) {
      // all loads of the chunk first; a clamped index and a 0/1 mask cover
      // the tail past dim
      float4 y[kSentBatch][kSentChunk], x[kSentChunk];
      float mk[kSentChunk];
#pragma unroll
      for (int c = 0; c < kSentChunk; ++c) {
        const int d = d0 + c * 64 + lane, dc = min(d, dim / 4 - 1);
        mk[c] = d < dim / 4 ? 1.f : 0.f;
#pragma unroll
        for (int u = 0; u < kSentBatch; ++u) y[u][c] = vj[u][dc];
        x[c] = ((const float4*)hv)[dc];
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of their uses
#pragma unroll
      for (int c = 0; c < kSentChunk; ++c) {
#pragma unroll
        for (int u = 0; u < kSentBatch; ++u) {
          const float4 a = y[u][c];
          dot[u] += mk[c] * (x[c].x * a.x + x[c].y * a.y + x[c].z * a.z + x[c].w * a.w);
          sj[u] += mk[c] * (a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kSentBatch; ++u) {
      const float dt = wave_sum(dot[u]), sn = wave_sum(sj[u]);
      if (j0 + u < n && ni > 0.f && sn > 0.f) {
        const float c = dt / (ni * sqrtf(sn));
        if (c > tau_s) best = fmaxf(best, c);
      }
    }
  }
  __syncthreads();  // red is reused
  if (lane == 0) red[w] = best;
  __syncthreads();
  if (tid == 0) {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) m = fmaxf(m, red[k]);
    *out = m > -INFINITY ? m : 0.f;
  }
}

// The sidecar's compaction: ids[j] <- ids[keep[j]] for every slice (order-
// preserving, the layout of the K/V compaction), -1 where keep[j] < 0. All
// reads go through LDS before any write, so the in-place gather is safe.
__global__ __launch_bounds__(kSentThreads) void compact_ids_kernel(Geom g, const int32_t* __restrict__ keep,
                                                                   int32_t* __restrict__ ids) {
  extern __shared__ __align__(16) int32_t stage[];
  const int slice = blockIdx.x, tid = threadIdx.x, B = g.budget;
  const int32_t* krow = keep + (size_t)slice * B;
  int32_t* irow = ids + (size_t)slice * g.capacity;
  for (int j = tid; j < B; j += kSentThreads) {
    const int k = krow[j];
    stage[j] = (k >= 0 && k < g.n_slots) ? irow[k] : -1;
  }
  __syncthreads();
  for (int j = tid; j < B; j += kSentThreads) irow[j] = stage[j];
}

int launch_sentence_penalty(const float* vectors, const int32_t* n_sent, int batch, int s_max, int dim, float tau_s,
                            float* penalty, void* stream) {
  if (batch == 0 || s_max == 0) return 0;
  // A sentence's row of later sentences is split over the waves of its work-
  // group. With few work-groups (fewer than two per compute unit) wider groups
  // finish the longest rows in fewer memory round trips; with many, the
  // narrow ones keep more rows in flight per compute unit.
  if ((long)s_max * batch < 2L * kCUs)
    RKV_LAUNCH(sentence_penalty_kernel<1024>, dim3(s_max, batch), dim3(1024), (size_t)dim * 4,
                       (hipStream_t)stream, vectors, n_sent, s_max, dim, tau_s, penalty);
  else
    RKV_LAUNCH(sentence_penalty_kernel<kSentThreads>, dim3(s_max, batch), dim3(kSentThreads), (size_t)dim * 4,
                       (hipStream_t)stream, vectors, n_sent, s_max, dim, tau_s, penalty);
  return 0;
}

int launch_compact_ids(const Geom& g, const int32_t* keep, int32_t* ids, void* stream) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  RKV_LAUNCH(compact_ids_kernel, dim3(slices), dim3(kSentThreads), (size_t)g.budget * 4,
                     (hipStream_t)stream, g, keep, ids);
  return 0;
}

}  // namespace rkv
