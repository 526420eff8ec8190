// K3 — redundancy Gram kernel with fused importance and row mean.
//
// Redundancy (R-KV notes page, yoonschallenge.tistory.com/1236, summary table
// row "redundancy computation"; Q&A part 2, cause 3: all-pairs key cosine)
// needs, for each valid token i, the number of newer tokens j > i whose
// cosine S_ij = k_i.k_j / (|k_i| |k_j|) exceeds tau (the protection test for
// the beta most recent similar tokens) and the mean cosine to the other
// tokens. The pairwise part is a dense contraction over head_dim = 128, run
// on the 32x32x16 bf16 MFMA with exact bf16 products and fp32 accumulation:
//
//   work unit  = column block I (128 older tokens, held in registers as MFMA
//                B fragments) x a segment of up to 6 row blocks of 64 newer
//                tokens (staged through LDS, double-buffered via registers),
//                starting at the diagonal, so only the upper triangle j >= i
//                is computed;
//   epilogue   = per element one multiply and one compare against
//                tau * |k_i| * |k_j| (norms from the stats kernel), counted
//                per column i in the lane that owns it; the N x N matrix never
//                leaves registers; per-column counts are combined across
//                waves in LDS and added to counts[] with integer atomics
//                (exact and order-independent).
//
// The first segment of each column block also computes, for its 128 keys,
// the importance (observation-query attention normalised by the per-row max
// and sum of exp reduced from the stats kernel's chunk partials, mean over
// the window, max over the GQA group) and the row mean of S through
// sum_{j != i} S_ij = khat_i . s - khat_i . khat_i with s the sum of unit keys.
#include "rkv_device.hpp"

namespace rkv {

constexpr int kGramThreads = 256;  // 4 waves: (column half) x (row half)

template <typename T>
__global__ __launch_bounds__(kGramThreads) void gram_kernel(Geom g, LayerPtrs k, const void* __restrict__ obs_q,
                                                            const int32_t* __restrict__ seq_start,
                                                            const float* __restrict__ norms,
                                                            const float* __restrict__ stats,
                                                            const float* __restrict__ ssum, float* __restrict__ importance,
                                                            float* __restrict__ rowmean, int32_t* __restrict__ counts) {
  constexpr int RB = kHeadDim * Elem<T>::kBytes;  // bytes per key row
  constexpr int RBP = RB + 16;                     // LDS row stride: +16 B keeps ds_read_b128 conflict-free
  constexpr int U4_ROW = RB / 16;
  constexpr int PER_T = kRowBlock * U4_ROW / kGramThreads;
  constexpr int kPStride = kColBlock + 1;
  static_assert(RKV_MAX_QROWS * kPStride * 4 <= 2 * kRowBlock * RBP, "importance scratch must fit the row buffers");

  __shared__ __align__(16) char jbuf[2][kRowBlock * RBP];
  __shared__ __align__(16) float nbuf[2][kRowBlock];
  __shared__ float qM[RKV_MAX_QROWS], qInvS[RKV_MAX_QROWS];
  __shared__ float svec[kHeadDim];
  __shared__ int cnt_x[kColBlock];

  const int units = gram_units(g.n_slots);
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = wid / units, u = wid % units;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;
  int I, jb_lo, jb_hi;
  if (!gram_unit_of(u, N, I, jb_lo, jb_hi)) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, col = lane & 31;
  const int cw = wave & 1;    // columns [64*cw, 64*cw + 64) of the column block
  const int jsub = wave >> 1;  // rows [32*jsub, 32*jsub + 32) of each row block
  const int col0 = I * kColBlock;
  const size_t srow = (size_t)slice * g.n_slots;
  const void* layer = k.p[l];

  // ---- column fragments (older tokens) and their thresholds tau * |k_i|
  Frag<T> bf[2];
  float tn[2];
#pragma unroll
  for (int is = 0; is < 2; ++is) {
    const int i = col0 + 64 * cw + 32 * is + col;
    if (i < N) {
      frag_load(bf[is], row_ptr<T>(layer, g, b, h, s0 + i) + hh * (RB / 2));
      const float n = norms[srow + s0 + i];
      tn[is] = g.tau * (n > 0.f ? n : 1.f);  // a zero key has cosine 0 with everything
    } else {
      frag_zero(bf[is]);
      tn[is] = 0.f;
    }
  }

  // ---- first segment: importance and row mean of the 128 column keys
  if (jb_lo == 0) {
    const int nch = chunks_of(g.n_slots), nvalid = chunks_of(N);
    if (tid < g.qrows) {
      const float* st = stats + (size_t)slice * nch * RKV_MAX_QROWS * 2;
      float M = -INFINITY;
      for (int c = 0; c < nvalid; ++c) M = fmaxf(M, st[(c * RKV_MAX_QROWS + tid) * 2]);
      float S = 0.f;
      for (int c = 0; c < nvalid; ++c) {
        const float mc = st[(c * RKV_MAX_QROWS + tid) * 2];
        if (mc > -INFINITY) S += st[(c * RKV_MAX_QROWS + tid) * 2 + 1] * __expf(mc - M);
      }
      qM[tid] = M;
      qInvS[tid] = 1.f / S;
    }
    if (tid < kHeadDim) {
      const float* sp = ssum + (size_t)slice * nch * kHeadDim + tid;
      float s = 0.f;
      for (int c = 0; c < nvalid; ++c) s += sp[(size_t)c * kHeadDim];
      svec[tid] = s;
    }
    __syncthreads();

    float* P = (float*)&jbuf[0][0];  // attention weights [query row][column], aliases the row buffers
    if (wave < 2) {
      const int ntile = (g.qrows + 31) >> 5;
      const char* qbase =
          (const char*)obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * RB;
      const float scale = 1.0f / sqrtf((float)kHeadDim);
      for (int t = 0; t < ntile; ++t) {
        const int qm = 32 * t + col;
        Frag<T> qf;
        if (qm < g.qrows)
          frag_load(qf, qbase + (size_t)qm * RB + hh * (RB / 2));
        else
          frag_zero(qf);
#pragma unroll
        for (int is = 0; is < 2; ++is) {
          f32x16 acc = {};
          mma_frag(acc, qf, bf[is]);
          const int c = 64 * cw + 32 * is + col;
          const int i = col0 + c;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = 32 * t + acc_row(r, hh);
            float pv = 0.f;
            if (m < g.qrows && i < N && i <= N - g.alpha + (m % g.alpha))
              pv = __expf(acc[r] * scale - qM[m]) * qInvS[m];
            P[m * kPStride + c] = pv;
          }
        }
      }
      // row mean of cosine through the sum of unit keys
#pragma unroll
      for (int is = 0; is < 2; ++is) {
        float dot = 0.f, ss = 0.f;
#pragma unroll
        for (int e = 0; e < 64; ++e) {
          const float x = frag_val(bf[is], e);
          dot = fmaf(x, svec[hh * 64 + e], dot);
          ss = fmaf(x, x, ss);
        }
        dot += __shfl_xor(dot, 32);
        ss += __shfl_xor(ss, 32);
        const int i = col0 + 64 * cw + 32 * is + col;
        if (hh == 0 && i < N) {
          const float nrm = sqrtf(ss);
          const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
          rowmean[srow + s0 + i] = (dot * inv - ss * inv * inv) / (float)(N - 1);
        }
      }
    }
    __syncthreads();
    if (tid < kColBlock && col0 + tid < N) {
      const int G = g.qrows / g.alpha;
      float best = 0.f;
      for (int gq = 0; gq < G; ++gq) {
        float s = 0.f;
        for (int t = 0; t < g.alpha; ++t) s += P[(gq * g.alpha + t) * kPStride + tid];
        best = fmaxf(best, s);
      }
      importance[srow + s0 + col0 + tid] = best / (float)g.alpha;
    }
    __syncthreads();
  }

  // ---- row-block loop: stage rows through LDS, MFMA, count similar pairs
  uint4 stg[PER_T];
  float stg_n = 0.f;
  auto prefetch = [&](int jb) {
    const int rbase = col0 + jb * kRowBlock;
#pragma unroll
    for (int q = 0; q < PER_T; ++q) {
      const int idx = q * kGramThreads + tid;
      const int jr = idx / U4_ROW, part = idx % U4_ROW;
      const int j = rbase + jr;
      stg[q] = j < N ? ((const uint4*)row_ptr<T>(layer, g, b, h, s0 + j))[part] : make_uint4(0, 0, 0, 0);
    }
    if (tid < kRowBlock) {
      const int j = rbase + tid;
      if (j < N) {
        const float n = norms[srow + s0 + j];
        stg_n = n > 0.f ? n : 1.f;
      } else {
        stg_n = __builtin_nanf("");  // rows past the slice never count
      }
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int q = 0; q < PER_T; ++q) {
      const int idx = q * kGramThreads + tid;
      const int jr = idx / U4_ROW, part = idx % U4_ROW;
      *(uint4*)(&jbuf[buf][jr * RBP + part * 16]) = stg[q];
    }
    if (tid < kRowBlock) nbuf[buf][tid] = stg_n;
  };

  int cnt[2] = {0, 0};
  prefetch(jb_lo);
  commit(0);
  __syncthreads();
  for (int jb = jb_lo; jb < jb_hi; ++jb) {
    const int cur = (jb - jb_lo) & 1;
    const bool more = jb + 1 < jb_hi;
    if (more) prefetch(jb + 1);

    Frag<T> af;
    frag_load(af, &jbuf[cur][(32 * jsub + col) * RBP + hh * (RB / 2)]);
    f32x16 acc0 = {}, acc1 = {};
    mma_frag(acc0, af, bf[0]);
    mma_frag(acc1, af, bf[1]);

    float nj[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 v = *(const float4*)&nbuf[cur][32 * jsub + 8 * a + 4 * hh];
      nj[4 * a + 0] = v.x;
      nj[4 * a + 1] = v.y;
      nj[4 * a + 2] = v.z;
      nj[4 * a + 3] = v.w;
    }
    if (jb * kRowBlock < kColBlock) {
      // row block overlaps the column block: count only j > i
      const int jrow0 = col0 + jb * kRowBlock + 32 * jsub;
      const int i0 = col0 + 64 * cw + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jrow0 + acc_row(r, hh);
        cnt[0] += (acc0[r] > tn[0] * nj[r]) && (j > i0);
        cnt[1] += (acc1[r] > tn[1] * nj[r]) && (j > i0 + 32);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        cnt[0] += acc0[r] > tn[0] * nj[r];
        cnt[1] += acc1[r] > tn[1] * nj[r];
      }
    }
    if (more) commit(cur ^ 1);
    __syncthreads();
  }

  // ---- combine the two row halves and the two waves sharing each column
#pragma unroll
  for (int is = 0; is < 2; ++is) cnt[is] += __shfl_xor(cnt[is], 32);
  if (jsub == 0 && hh == 0) {
    cnt_x[64 * cw + col] = cnt[0];
    cnt_x[64 * cw + 32 + col] = cnt[1];
  }
  __syncthreads();
  if (jsub == 1 && hh == 0) {
#pragma unroll
    for (int is = 0; is < 2; ++is) {
      const int c = 64 * cw + 32 * is + col;
      const int total = cnt[is] + cnt_x[c];
      if (col0 + c < N && total) atomicAdd(&counts[srow + s0 + col0 + c], total);
    }
  }
}

// rbar = 0 for protected tokens (fewer than beta newer similar tokens), else
// the row mean of cosine; written for the valid slots of evicting sequences.
__global__ void redundancy_kernel(Geom g, const int32_t* __restrict__ seq_start, const int32_t* __restrict__ counts,
                                  const float* __restrict__ rowmean, float* __restrict__ redundancy) {
  const int slice = blockIdx.y;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (N <= g.budget || j >= N) return;
  const size_t idx = (size_t)slice * g.n_slots + s0 + j;
  redundancy[idx] = counts[idx] < g.beta ? 0.f : rowmean[idx];
}

int launch_gram(const Geom& g, int dtype, const LayerPtrs& k, const void* obs_q, const int32_t* seq_start,
                const float* norms, const float* stats, const float* ssum, float* importance, float* rowmean,
                int32_t* counts, void* stream) {
  const int slices = g.L * g.batch * g.H;
  const int blocks = slices * gram_units(g.n_slots);
  if (blocks == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == RKV_BF16)
    hipLaunchKernelGGL(gram_kernel<bf16_t>, dim3(blocks), dim3(kGramThreads), 0, s, g, k, obs_q, seq_start, norms,
                       stats, ssum, importance, rowmean, counts);
  else
    hipLaunchKernelGGL(gram_kernel<float>, dim3(blocks), dim3(kGramThreads), 0, s, g, k, obs_q, seq_start, norms,
                       stats, ssum, importance, rowmean, counts);
  return (int)hipGetLastError();
}

int launch_redundancy(const Geom& g, const int32_t* seq_start, const int32_t* counts, const float* rowmean,
                      float* redundancy, void* stream) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0 || g.n_slots == 0) return 0;
  dim3 grid((g.n_slots + 255) / 256, slices);
  hipLaunchKernelGGL(redundancy_kernel, grid, dim3(256), 0, (hipStream_t)stream, g, seq_start, counts, rowmean,
                     redundancy);
  return (int)hipGetLastError();
}

}  // namespace rkv
