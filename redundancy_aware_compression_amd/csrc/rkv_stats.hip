// K1 — per-chunk statistics of one slice's keys, the bandwidth-bound first
// pass of R-KV scoring.
//
// Importance (R-KV notes page, yoonschallenge.tistory.com/1236, summary table
// row "importance computation") needs, for every observation query row
// m = g*alpha + t, the maximum and the sum of exp over the causal softmax
// row; redundancy needs key norms (Q&A part 2, cause 3: key normalisation)
// and, through the identity sum_{j != i} S_ij = khat_i . s - khat_i . khat_i,
// the sum s of unit keys. One work-group reads one chunk of 128 keys once
// from HBM and emits:
//   norms[slot]                       ||k_j|| in fp32 from exact bf16 values
//   stats[chunk][m] = (max, sum exp)  of q_m . k_j / sqrt(D) over the chunk
//   ssum[chunk][d]                    sum over the chunk of k_j[d] / ||k_j||
// and zeroes counts[slot] for the Gram kernel's atomic accumulation.
// Logits use the 32x32 bf16 MFMA (32 keys x up to 64 query rows per wave).
#include "rkv_device.hpp"

namespace rkv {

constexpr int kStatsThreads = 256;  // 4 waves x 32 keys = kChunk

template <typename T>
__global__ __launch_bounds__(kStatsThreads) void stats_kernel(Geom g, LayerPtrs k, const void* __restrict__ obs_q,
                                                              const int32_t* __restrict__ seq_start,
                                                              float* __restrict__ norms, int32_t* __restrict__ counts,
                                                              float* __restrict__ stats, float* __restrict__ ssum) {
  __shared__ float lg[RKV_MAX_QROWS][kChunk + 1];  // masked logits of the chunk
  __shared__ float red[4][kHeadDim];              // per-wave sums of unit keys

  const int nchunk = chunks_of(g.n_slots);
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = wid / nchunk, chunk = wid % nchunk;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget || chunk * kChunk >= N) return;  // uniform over the block

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, col = lane & 31;
  const int j = chunk * kChunk + wave * 32 + col;  // key index within the slice
  const bool valid = j < N;
  const size_t srow = (size_t)slice * g.n_slots;

  Frag<T> kf;
  if (valid)
    frag_load(kf, row_ptr<T>(k.p[l], g, b, h, s0 + j) + hh * 64 * Elem<T>::kBytes);
  else
    frag_zero(kf);

  // ---- norm of key j (both half-lanes hold 64 dims each)
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    const float x = frag_val(kf, e);
    ss = fmaf(x, x, ss);
  }
  ss += __shfl_xor(ss, 32);
  const float nrm = sqrtf(ss);
  const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
  if (valid && hh == 0) {
    norms[srow + s0 + j] = nrm;
    counts[srow + s0 + j] = 0;
  }

  // ---- sum of unit keys over the wave's 32 keys: butterfly reduce-scatter
  // over the 32 lanes of each half; lane `col` ends with dims 2*col, 2*col+1
  // of its half.
  {
    float v[64];
#pragma unroll
    for (int e = 0; e < 64; ++e) v[e] = frag_val(kf, e) * inv;
#pragma unroll
    for (int step = 0; step < 5; ++step) {
      const int mask = 16 >> step;
      const int half = 32 >> step;  // values kept after this step
      const bool up = (col & mask) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float keep_v = up ? v[half + i] : v[i];
        const float send_v = up ? v[i] : v[half + i];
        v[i] = keep_v + __shfl_xor(send_v, mask);
      }
    }
    red[wave][hh * 64 + 2 * col] = v[0];
    red[wave][hh * 64 + 2 * col + 1] = v[1];
  }

  // ---- logits of the chunk for every observation query row
  const int ntile = (g.qrows + 31) >> 5;
  const char* qbase = (const char*)obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows *
                                               (kHeadDim * Elem<T>::kBytes);
  const float scale = 1.0f / sqrtf((float)kHeadDim);
  for (int t = 0; t < ntile; ++t) {
    const int qm = 32 * t + col;
    Frag<T> qf;
    if (qm < g.qrows)
      frag_load(qf, qbase + (size_t)qm * (kHeadDim * Elem<T>::kBytes) + hh * 64 * Elem<T>::kBytes);
    else
      frag_zero(qf);
    f32x16 acc = {};
    mma_frag(acc, qf, kf);  // rows: query rows, columns: keys
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * t + acc_row(r, hh);
      const int pos = N - g.alpha + (m % g.alpha);  // position of the query's token
      const bool ok = valid && m < g.qrows && j <= pos;
      if (m < RKV_MAX_QROWS) lg[m][wave * 32 + col] = ok ? acc[r] * scale : -INFINITY;
    }
  }
  __syncthreads();

  // ---- chunk max and sum of exp per query row: 4 threads per row
  {
    const int m = tid >> 2, q = tid & 3;
    float mx = -INFINITY;
    if (m < g.qrows)
      for (int c = q * 32; c < q * 32 + 32; ++c) mx = fmaxf(mx, lg[m][c]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    float sum = 0.f;
    if (m < g.qrows && mx > -INFINITY)
      for (int c = q * 32; c < q * 32 + 32; ++c) sum += __expf(lg[m][c] - mx);
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    if (m < g.qrows && q == 0) {
      float* st = stats + (((size_t)slice * nchunk + chunk) * RKV_MAX_QROWS + m) * 2;
      st[0] = mx;
      st[1] = sum;
    }
  }
  if (tid < kHeadDim)
    ssum[((size_t)slice * nchunk + chunk) * kHeadDim + tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
}

int launch_stats(const Geom& g, int dtype, const LayerPtrs& k, const void* obs_q, const int32_t* seq_start,
                 float* norms, int32_t* counts, float* stats, float* ssum, void* stream) {
  const int slices = g.L * g.batch * g.H;
  const int blocks = slices * chunks_of(g.n_slots);
  if (blocks == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == RKV_BF16)
    hipLaunchKernelGGL(stats_kernel<bf16_t>, dim3(blocks), dim3(kStatsThreads), 0, s, g, k, obs_q, seq_start,
                       norms, counts, stats, ssum);
  else
    hipLaunchKernelGGL(stats_kernel<float>, dim3(blocks), dim3(kStatsThreads), 0, s, g, k, obs_q, seq_start,
                       norms, counts, stats, ssum);
  return (int)hipGetLastError();
}

}  // namespace rkv
