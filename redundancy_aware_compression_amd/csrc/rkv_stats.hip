// K1 — per-chunk statistics of one slice's keys, the bandwidth-bound first
// pass of R-KV scoring.
//
// Importance (R-KV notes page, yoonschallenge.tistory.com/1236, summary table
// row "importance computation") needs, for every observation query row
// m = g*alpha + t, the maximum and the sum of exp over the causal softmax
// row; redundancy needs key norms (Q&A part 2, cause 3: key normalisation)
// and, through the identity sum_{j != i} S_ij = khat_i . s - khat_i . khat_i,
// the sum s of unit keys. The keys are read once from HBM, in chunks of 128,
// and the pass emits:
//   norms[slot]                      ||k_j|| in fp32 from exact bf16 values
//                                    (-1 for a zero key)
//   stats[part][m] = (max, sum exp)  of q_m . k_j / sqrt(D) over the part's keys
//   ssum[part][d]                    sum over the part's keys of k_j[d] / ||k_j||
// and zeroes counts[slot] for the Gram kernel's atomic accumulation. A
// work-group walks a contiguous range of chunks of one slice, prefetching the
// next chunk's keys while it works on the current one, and merges the chunk
// statistics into running values, so it writes one partial per range.
// Logits use the 32x32 bf16 MFMA (32 keys x up to 64 query rows per wave).
#include "rkv_device.hpp"

namespace rkv {

constexpr int kStatsThreads = 256;  // 4 waves x 32 keys = kChunk

// One butterfly reduce-scatter pass over dims [32*PASS, 32*PASS + 32) of the
// lane's half-row, summed over the 32 lanes that share the half: every
// register index is a compile-time constant.
template <int PASS, typename T>
__device__ inline void unit_key_pass(const Frag<T>& kf, float inv, int col, float* out) {
  float v[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = frag_val(kf, 32 * PASS + e) * inv;
#pragma unroll
  for (int step = 0; step < 5; ++step) {
    const int mask = 16 >> step;
    const int half = 16 >> step;  // values kept after this step
    const bool up = (col & mask) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep_v = up ? v[half + i] : v[i];
      const float send_v = up ? v[i] : v[half + i];
      v[i] = keep_v + __shfl_xor(send_v, mask);
    }
  }
  out[32 * PASS + col] = v[0];
}

// Chunks of 128 keys handled by work-group `part` of a slice split `split` ways.
__device__ inline void part_range(int n_slots, int N, int split, int part, int& c_lo, int& c_hi) {
  const int cps = (chunks_of(n_slots) + split - 1) / split;
  c_lo = part * cps;
  c_hi = min(chunks_of(N), c_lo + cps);
}

template <typename T>
__global__ __launch_bounds__(kStatsThreads) void stats_kernel(Geom g, LayerPtrs k, const void* __restrict__ obs_q,
                                                              const int32_t* __restrict__ seq_start,
                                                              float* __restrict__ norms, int32_t* __restrict__ counts,
                                                              float* __restrict__ stats, float* __restrict__ ssum,
                                                              int split) {
  constexpr int RB = kHeadDim * Elem<T>::kBytes;
  constexpr int RBP = RB + 16;  // padded LDS rows: conflict-free ds_read_b128
  constexpr int U4_ROW = RB / 16;
  __shared__ __align__(16) char qs[RKV_MAX_QROWS * RBP];             // observation queries
  __shared__ __align__(16) float lg[RKV_MAX_QROWS][kChunk + 4];  // masked logits of one chunk
  __shared__ float red[4][kHeadDim];                              // per-wave sums of unit keys

  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = wid / split, part = wid % split;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;  // uniform over the block
  int c_lo, c_hi;
  part_range(g.n_slots, N, split, part, c_lo, c_hi);
  if (c_lo >= c_hi) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, col = lane & 31;
  const size_t srow = (size_t)slice * g.n_slots;
  const void* layer = k.p[l];

  auto load_keys = [&](Frag<T>& f, int c) {
    const int j = c * kChunk + wave * 32 + col;
    if (j < N)
      frag_load(f, row_ptr<T>(layer, g, b, h, s0 + j) + hh * (RB / 2));
    else
      frag_zero(f);
  };
  Frag<T> kf;
  load_keys(kf, c_lo);

  // observation queries -> LDS once per work-group (rows past G*alpha are zero)
  {
    const char* qbase = (const char*)obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * RB;
    for (int idx = tid; idx < RKV_MAX_QROWS * U4_ROW; idx += kStatsThreads) {
      const int m = idx / U4_ROW, part16 = idx % U4_ROW;
      *(uint4*)&qs[m * RBP + part16 * 16] =
          m < g.qrows ? ((const uint4*)(qbase + (size_t)m * RB))[part16] : make_uint4(0, 0, 0, 0);
    }
  }
  const int ntile = (g.qrows + 31) >> 5;
  const float scale = 1.0f / sqrtf((float)kHeadDim);
  const int rm = tid >> 2, rq = tid & 3;  // row-reduction role: 4 threads per query row
  float runM = -INFINITY, runS = 0.f;     // running softmax statistics of row rm
  float runSum = 0.f;                     // running sum of unit keys, dim tid (tid < 128)
  __syncthreads();

  for (int c = c_lo; c < c_hi; ++c) {
    Frag<T> kn;
    if (c + 1 < c_hi) load_keys(kn, c + 1);  // prefetch: in flight during this chunk
    const int j = c * kChunk + wave * 32 + col;
    const bool valid = j < N;

    // ---- norm of key j (each half-lane holds 64 dims)
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
      norms[srow + s0 + j] = nrm > 0.f ? nrm : -1.f;  // -1 marks a zero key
      counts[srow + s0 + j] = 0;
    }

    // ---- masked logits q_m . k_j / sqrt(D) of the chunk
    for (int t = 0; t < ntile; ++t) {
      Frag<T> qf;
      frag_load(qf, &qs[(32 * t + col) * RBP + hh * (RB / 2)]);
      f32x16 acc = {};
      mma_frag(acc, qf, kf);  // rows: query rows, columns: keys
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * t + acc_row(r, hh);
        const int pos = N - g.alpha + (m % g.alpha);  // position of the query's token
        const bool ok = valid && m < g.qrows && j <= pos;
        lg[m][wave * 32 + col] = ok ? acc[r] * scale : -INFINITY;
      }
    }

    // ---- sum of unit keys over the wave's 32 keys
    unit_key_pass<0>(kf, inv, col, &red[wave][hh * 64]);
    unit_key_pass<1>(kf, inv, col, &red[wave][hh * 64]);
    __syncthreads();

    // ---- chunk max / sum of exp per query row, merged into the running pair
    if (rm < ntile * 32) {
      float x[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = *(const float4*)&lg[rm][rq * 32 + 4 * q];
        x[4 * q] = v.x;
        x[4 * q + 1] = v.y;
        x[4 * q + 2] = v.z;
        x[4 * q + 3] = v.w;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < 32; ++q) mx = fmaxf(mx, x[q]);
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      float sum = 0.f;
      if (mx > -INFINITY) {
#pragma unroll
        for (int q = 0; q < 32; ++q) sum += __expf(x[q] - mx);
      }
      sum += __shfl_xor(sum, 1);
      sum += __shfl_xor(sum, 2);
      if (mx > -INFINITY) {
        const float M = fmaxf(runM, mx);
        runS = (runM > -INFINITY ? runS * __expf(runM - M) : 0.f) + sum * __expf(mx - M);
        runM = M;
      }
    }
    if (tid < kHeadDim) runSum += red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    __syncthreads();  // lg and red are rewritten by the next chunk
    if (c + 1 < c_hi) kf = kn;
  }

  if (rm < g.qrows && rq == 0) {
    float* st = stats + (((size_t)slice * chunks_of(g.n_slots) + part) * RKV_MAX_QROWS + rm) * 2;
    st[0] = runM;
    st[1] = runS;
  }
  if (tid < kHeadDim) ssum[((size_t)slice * chunks_of(g.n_slots) + part) * kHeadDim + tid] = runSum;
}

// K2 — per slice, reduces the chunk partials to the final statistics the
// Gram kernel needs: rowstat[m] = (max, 1 / sum of exp) of every query row's
// causal softmax, and svec = sum over all valid keys of unit keys.
__global__ __launch_bounds__(256) void reduce_stats_kernel(Geom g, const int32_t* __restrict__ seq_start,
                                                           const float* __restrict__ stats,
                                                           const float* __restrict__ ssum,
                                                           float* __restrict__ rowstat, float* __restrict__ svec,
                                                           int split) {
  const int slice = blockIdx.x;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;
  const int nch = chunks_of(g.n_slots);
  int nparts = 0;  // parts whose chunk range is non-empty
  for (int p = 0; p < split; ++p) {
    int lo, hi;
    part_range(g.n_slots, N, split, p, lo, hi);
    nparts += lo < hi;
  }
  const int tid = threadIdx.x;
  // 4 threads per query row, each over every 4th part
  {
    const int m = tid >> 2, q = tid & 3;
    const float* st = stats + (size_t)slice * nch * RKV_MAX_QROWS * 2;
    float M = -INFINITY;
    if (m < g.qrows) {
#pragma unroll 4
      for (int c = q; c < nparts; c += 4) M = fmaxf(M, st[(c * RKV_MAX_QROWS + m) * 2]);
    }
    M = fmaxf(M, __shfl_xor(M, 1));
    M = fmaxf(M, __shfl_xor(M, 2));
    float S = 0.f;
    if (m < g.qrows) {
#pragma unroll 4
      for (int c = q; c < nparts; c += 4) {
        const float mc = st[(c * RKV_MAX_QROWS + m) * 2];
        const float sc = st[(c * RKV_MAX_QROWS + m) * 2 + 1];
        if (mc > -INFINITY) S += sc * __expf(mc - M);
      }
    }
    S += __shfl_xor(S, 1);
    S += __shfl_xor(S, 2);
    if (q == 0) {  // rows past the group's queries get (0, 0): their weights vanish
      rowstat[((size_t)slice * RKV_MAX_QROWS + m) * 2] = m < g.qrows ? M : 0.f;
      rowstat[((size_t)slice * RKV_MAX_QROWS + m) * 2 + 1] = m < g.qrows ? 1.f / S : 0.f;
    }
  }
  // 2 threads per dimension, each over every other part
  {
    const int d = tid >> 1, q = tid & 1;
    const float* sp = ssum + (size_t)slice * nch * kHeadDim + d;
    float acc = 0.f;
#pragma unroll 4
    for (int c = q; c < nparts; c += 2) acc += sp[(size_t)c * kHeadDim];
    acc += __shfl_xor(acc, 1);
    if (q == 0) svec[(size_t)slice * kHeadDim + d] = acc;
  }
}

// Work-groups per slice for the statistics pass: enough to give every CU
// about two, each walking a contiguous range of chunks.
inline int stats_split(const Geom& g) {
  const int slices = g.L * g.batch * g.H;
  const int want = (512 + slices - 1) / slices;
  const int nch = chunks_of(g.n_slots);
  return want < 1 ? 1 : (want > nch ? nch : want);
}

int launch_reduce_stats(const Geom& g, const int32_t* seq_start, const float* stats, const float* ssum,
                        float* rowstat, float* svec, void* stream) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  hipLaunchKernelGGL(reduce_stats_kernel, dim3(slices), dim3(256), 0, (hipStream_t)stream, g, seq_start, stats, ssum,
                     rowstat, svec, stats_split(g));
  return (int)hipGetLastError();
}

int launch_stats(const Geom& g, int dtype, const LayerPtrs& k, const void* obs_q, const int32_t* seq_start,
                 float* norms, int32_t* counts, float* stats, float* ssum, void* stream) {
  const int slices = g.L * g.batch * g.H;
  const int split = stats_split(g);
  const int blocks = slices * split;
  if (blocks == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == RKV_BF16)
    hipLaunchKernelGGL(stats_kernel<bf16_t>, dim3(blocks), dim3(kStatsThreads), 0, s, g, k, obs_q, seq_start,
                       norms, counts, stats, ssum, split);
  else
    hipLaunchKernelGGL(stats_kernel<float>, dim3(blocks), dim3(kStatsThreads), 0, s, g, k, obs_q, seq_start,
                       norms, counts, stats, ssum, split);
  return (int)hipGetLastError();
}

}  // namespace rkv
