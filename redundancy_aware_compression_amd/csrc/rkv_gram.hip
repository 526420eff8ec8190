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
//                B fragments) x every row block of 64 newer tokens from the
//                diagonal to the end of the slice, so only the upper triangle
//                j >= i is computed; row blocks and their norms stream through
//                a 4-deep LDS ring filled by direct buffer-to-LDS loads (no
//                staging registers, hardware range checks past the slice), a
//                stage being refilled as soon as every wave is past it; LDS
//                rows are XOR-swizzled in 16-byte slots so the MFMA operand
//                reads are conflict-free;
//   epilogue   = per element one fma, tau*|k_i|*|k_j| - G_ij, whose sign bit
//                (norms from the stats kernel) is added to the count of
//                column i in the lane that owns it; the N x N matrix never
//                leaves registers; per-column counts are combined across
//                waves in LDS and added to counts[] with integer atomics
//                (exact and order-independent).
//
// Each work unit also computes, for its 128 column keys,
// the importance (observation-query attention normalised by each query row's
// max and sum of exp from the statistics pass, mean over the window, max over
// the GQA group) and the row mean of S through
// sum_{j != i} S_ij = khat_i . s - khat_i . khat_i with s the sum of unit keys.
#include "rkv_device.hpp"

namespace rkv {

constexpr int kGramThreads = 256;  // 4 waves: (column half) x (row half)

// s_waitcnt immediate for vmcnt(v), other counters unconstrained (gfx9 encoding).
__device__ constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

// Waits until at most `later` stages of PER direct-to-LDS loads each, issued
// by this wave after the awaited one, are still in flight.
template <int PER>
__device__ inline void wait_later_stages(int later) {
  static_assert(kStages <= 4 && 3 * PER < 64, "vmcnt has 6 bits");
  switch (later) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PER)); break;
  }
}

template <typename T>
struct Stage {
  static constexpr int RB = kHeadDim * Elem<T>::kBytes;  // bytes per key row
  static constexpr int SLOTS = RB / 16;                   // 16-byte slots per row
  static constexpr int PER_WAVE = SLOTS / 4;              // 1 KB direct loads per wave per row block
  static constexpr int PER = PER_WAVE + 1;                // + one norm load
  static constexpr int BYTES = kRowBlock * RB;
};

// Issues the direct-to-LDS loads of one row block: row r of the block lands
// at st_rows + r*RB with 16-byte slot p holding the row's bytes
// [16*(p ^ (r & 15)), +16); its norm lands at st_norms[r]. voff[q] is the
// lane's stage-invariant byte offset for load q; the block's first row
// enters through the scalar offset. Rows past the slice read as zeros.
template <typename T>
__device__ inline void issue_stage(char* st_rows, float* st_norms, __amdgpu_buffer_rsrc_t rk,
                                   __amdgpu_buffer_rsrc_t rn, const uint32_t* voff, uint32_t nvoff, int rbase,
                                   int wave, int lane) {
  using S = Stage<T>;
#pragma unroll
  for (int q = 0; q < S::PER_WAVE; ++q)
    buf_to_lds16(rk, st_rows + (wave * S::PER_WAVE + q) * 1024, voff[q], (uint32_t)rbase * S::RB);
  if (lane < 16) buf_to_lds4(rn, st_norms + wave * 16, nvoff, (uint32_t)rbase * 4);
}

// MFMA A fragment of staged row R (the lane's half hh) from a swizzled stage.
template <typename T>
__device__ inline void frag_from_stage(Frag<T>& f, const char* st_rows, int R, int hh) {
  using S = Stage<T>;
  const char* row = st_rows + R * S::RB;
  const int sw = R & 15;
#pragma unroll
  for (int s = 0; s < Frag<T>::kU4; ++s) f.v[s] = *(const uint4*)(row + (((hh * (S::SLOTS / 2) + s) ^ sw) * 16));
}

template <typename T>
__global__ __launch_bounds__(kGramThreads) void gram_kernel(Geom g, LayerPtrs k, const void* __restrict__ obs_q,
                                                            const int32_t* __restrict__ seq_start,
                                                            const float* __restrict__ norms,
                                                            const float* __restrict__ rowstat,
                                                            const float* __restrict__ svec,
                                                            float* __restrict__ importance,
                                                            float* __restrict__ rowmean, int32_t* __restrict__ counts) {
  using S = Stage<T>;
  constexpr int RB = S::RB;
  constexpr int kPStride = kColBlock + 1;
  static_assert(RKV_MAX_QROWS * kPStride * 4 <= kStages * S::BYTES, "importance scratch must fit the stages");

  __shared__ __align__(16) char rows_lds[kStages * S::BYTES];
  __shared__ __align__(16) float nrm_lds[kStages][kRowBlock];
  __shared__ __align__(16) float qM[RKV_MAX_QROWS];
  __shared__ __align__(16) float qInvS[RKV_MAX_QROWS];
  __shared__ __align__(16) int qPos[RKV_MAX_QROWS];
  __shared__ __align__(16) float sv[kHeadDim];
  __shared__ int cnt_x[kColBlock];

  const int units = gram_units(g.n_slots);
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = wid / units, u = wid % units;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;
  const int I = u;
  if (I * kColBlock >= N) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, col = lane & 31;
  const int cw = wave & 1;    // columns [64*cw, 64*cw + 64) of the column block
  const int jsub = wave >> 1;  // rows [32*jsub, 32*jsub + 32) of each row block
  const int col0 = I * kColBlock;
  const size_t srow = (size_t)slice * g.n_slots;
  const float* norms_row = norms + srow + s0;
  const void* layer = k.p[l];
  const int nb = gram_row_blocks(N, I);

  // the slice's valid rows and norms as range-checked buffers
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(row_ptr<T>(layer, g, b, h, s0), (uint32_t)N * RB);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(norms_row, (uint32_t)N * 4);

  // ---- column fragments (older tokens) and their thresholds tau * |k_i|
  Frag<T> bf[2];
  float nrm_i[2], tn[2];
#pragma unroll
  for (int is = 0; is < 2; ++is) {
    const int i = col0 + 64 * cw + 32 * is + col;
    frag_load_buf(bf[is], rk, (uint32_t)i * RB + hh * (RB / 2));  // zeros past the slice
    nrm_i[is] = i < N ? norms_row[i] : 0.f;
    tn[is] = g.tau * fabsf(nrm_i[is]);  // a zero key (norm -1) compares as a unit-norm key with G = 0
  }

  // stage-invariant per-lane offsets of the row-block loads
  uint32_t voff[S::PER_WAVE];
#pragma unroll
  for (int q = 0; q < S::PER_WAVE; ++q) {
    const int flat = (wave * S::PER_WAVE + q) * 64 + lane;
    const int r = flat / S::SLOTS, p = flat % S::SLOTS;
    voff[q] = (uint32_t)r * RB + (uint32_t)(p ^ (r & 15)) * 16;
  }
  const uint32_t nvoff = (uint32_t)(wave * 16 + lane) * 4;
  auto issue = [&](int bi) {  // row block bi of this column block into stage bi % kStages
    issue_stage<T>(rows_lds + (bi % kStages) * S::BYTES, nrm_lds[bi % kStages], rk, rn, voff, nvoff,
                   col0 + bi * kRowBlock, wave, lane);
  };

  // ---- importance and row mean of the 128 column keys
  {
    if (tid < RKV_MAX_QROWS) {
      const bool row_ok = tid < g.qrows;
      qM[tid] = row_ok ? rowstat[((size_t)slice * RKV_MAX_QROWS + tid) * 2] : 0.f;
      qInvS[tid] = row_ok ? rowstat[((size_t)slice * RKV_MAX_QROWS + tid) * 2 + 1] : 0.f;
      qPos[tid] = row_ok ? N - g.alpha + tid % g.alpha : -1;  // last key the row's query attends to
    }
    if (tid < kHeadDim) sv[tid] = svec[(size_t)slice * kHeadDim + tid];
    __syncthreads();

    float* P = (float*)rows_lds;  // attention weights [query row][column], aliases the stages
    if (wave < 2) {
      const int ntile = (g.qrows + 31) >> 5;
      const char* qbase = (const char*)obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * RB;
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
            const float pv = __expf(acc[r] * scale - qM[m]) * qInvS[m];
            P[m * kPStride + c] = (i <= qPos[m] && i < N) ? pv : 0.f;
          }
        }
      }
      // row mean of cosine through the sum of unit keys:
      // sum_{j != i} S_ij = khat_i . s - khat_i . khat_i
      const float inv_nm1 = 1.f / (float)(N - 1);
#pragma unroll
      for (int is = 0; is < 2; ++is) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 64; ++e) dot = fmaf(frag_val(bf[is], e), sv[hh * 64 + e], dot);
        dot += __shfl_xor(dot, 32);
        const int i = col0 + 64 * cw + 32 * is + col;
        if (hh == 0 && i < N) {
          const float inv = nrm_i[is] > 0.f ? 1.f / nrm_i[is] : 0.f;
          const float self = nrm_i[is] > 0.f ? 1.f : 0.f;
          rowmean[srow + s0 + i] = (dot * inv - self) * inv_nm1;
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
    __syncthreads();  // P is overwritten by the stages
  }
  for (int bi = 0; bi < nb && bi < kStages; ++bi) issue(bi);

  // ---- row blocks in arrival order: MFMA, then count similar pairs
  uint32_t cnt[2] = {0u, 0u};
  const int i0 = col0 + 64 * cw + col;  // column of cnt[0]; cnt[1] is column i0 + 32
  for (int bi = 0; bi < nb; ++bi) {
    // blocks issued so far: the first kStages, then one refill per iteration
    // from iteration 1 on (block bi' - 1 + kStages in iteration bi'), so the
    // last one issued before this wait is max(kStages - 1, bi + kStages - 2)
    const int last = min(nb - 1, max(kStages - 1, bi + kStages - 2));
    wait_later_stages<S::PER>(last - bi);
    __syncthreads();  // every wave's share of row block bi is in LDS, and every
                      // wave is done with block bi - 1, whose stage is free
    if (bi >= 1 && bi - 1 + kStages < nb) issue(bi - 1 + kStages);
    const int jb = bi;
    const int stg = bi % kStages;
    const char* st = rows_lds + stg * S::BYTES;

    Frag<T> af;
    frag_from_stage(af, st, 32 * jsub + col, hh);
    f32x16 acc0 = {}, acc1 = {};
    mma_frag(acc0, af, bf[0]);
    mma_frag(acc1, af, bf[1]);

    float nj[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 v = *(const float4*)&nrm_lds[stg][32 * jsub + 8 * a + 4 * hh];
      nj[4 * a + 0] = fabsf(v.x);
      nj[4 * a + 1] = fabsf(v.y);
      nj[4 * a + 2] = fabsf(v.z);
      nj[4 * a + 3] = fabsf(v.w);
    }
    // similar iff G_ij > tau |k_i| |k_j|, i.e. iff d = tau|k_i| |k_j| - G_ij is
    // negative: one fma per element, then its sign bit is counted (no
    // compare / carry chain)
    const int rbase = col0 + jb * kRowBlock;
    if (jb * kRowBlock < kColBlock || rbase + kRowBlock > N) {
      // overlaps the column block (count only j > i) or runs past the slice
      const int jrow0 = rbase + 32 * jsub;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jrow0 + acc_row(r, hh);
        const uint32_t s0b = __float_as_uint(fmaf(tn[0], nj[r], -acc0[r])) >> 31;
        const uint32_t s1b = __float_as_uint(fmaf(tn[1], nj[r], -acc1[r])) >> 31;
        cnt[0] += (j > i0 && j < N) ? s0b : 0u;
        cnt[1] += (j > i0 + 32 && j < N) ? s1b : 0u;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        cnt[0] += (__float_as_uint(fmaf(tn[0], nj[r], -acc0[r])) >> 31) +
                  (__float_as_uint(fmaf(tn[0], nj[r + 1], -acc0[r + 1])) >> 31);
        cnt[1] += (__float_as_uint(fmaf(tn[1], nj[r], -acc1[r])) >> 31) +
                  (__float_as_uint(fmaf(tn[1], nj[r + 1], -acc1[r + 1])) >> 31);
      }
    }
  }

  // ---- combine the two row halves and the two waves sharing each column
#pragma unroll
  for (int is = 0; is < 2; ++is) cnt[is] += __shfl_xor(cnt[is], 32);
  if (jsub == 0 && hh == 0) {
    cnt_x[64 * cw + col] = (int)cnt[0];
    cnt_x[64 * cw + 32 + col] = (int)cnt[1];
  }
  __syncthreads();
  if (jsub == 1 && hh == 0) {
#pragma unroll
    for (int is = 0; is < 2; ++is) {
      const int c = 64 * cw + 32 * is + col;
      const int total = (int)cnt[is] + cnt_x[c];
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
                const float* norms, const float* rowstat, const float* svec, float* importance, float* rowmean,
                int32_t* counts, void* stream) {
  const int slices = g.L * g.batch * g.H;
  const int blocks = slices * gram_units(g.n_slots);
  if (blocks == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == RKV_BF16)
    hipLaunchKernelGGL(gram_kernel<bf16_t>, dim3(blocks), dim3(kGramThreads), 0, s, g, k, obs_q, seq_start, norms,
                       rowstat, svec, importance, rowmean, counts);
  else
    hipLaunchKernelGGL(gram_kernel<float>, dim3(blocks), dim3(kGramThreads), 0, s, g, k, obs_q, seq_start, norms,
                       rowstat, svec, importance, rowmean, counts);
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
