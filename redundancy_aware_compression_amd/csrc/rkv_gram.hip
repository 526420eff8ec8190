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
//   work unit  = column group g of a slice: the 64-token row blocks
//                4g .. 4g+3 are the columns (older tokens) of its 4 waves,
//                64 each, held in registers as MFMA B fragments; every row
//                block from 4g to the end of the slice streams once through
//                an LDS ring filled by direct buffer-to-LDS loads (no staging
//                registers, hardware range checks past the slice), a stage
//                being refilled as soon as every wave is past it; LDS rows
//                are XOR-swizzled in 16-byte slots so the MFMA operand reads
//                are conflict-free. Wave w has nothing to do before block
//                4g+w, which holds its own columns: it takes its B fragments
//                and norms from the ring there (no separate column loads),
//                so about the upper triangle j >= i is computed; the ring is
//                small enough for two groups per CU;
//   epilogue   = per element one fma, tau*|k_i|*|k_j| - G_ij, whose sign bit
//                (norms from the stats kernel) is added to the count of
//                column i in the lane that owns it; the N x N matrix never
//                leaves registers; each column belongs to one lane, which
//                stores its count (no atomics).
//
// After the last row block every wave computes, for its columns, the
// importance (observation-query attention normalised by each query row's max
// and sum of exp from the statistics pass, mean over the window, max over
// the GQA group; the window sums are taken in registers) and the row mean of
// S through sum_{j != i} S_ij = khat_i . s - khat_i . khat_i with s the sum
// of unit keys.
#include "rkv_device.hpp"

namespace rkv {

constexpr int kGramThreads = kGramWaves * 64;
static_assert(kGramThreads >= kHeadDim && kGramThreads >= RKV_MAX_QROWS, "per-slice constants: one thread each");

// s_waitcnt immediate for vmcnt(v), other counters unconstrained (gfx9 encoding).
__device__ constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

template <typename T>
struct Stage {
  static constexpr int RB = kHeadDim * Elem<T>::kBytes;      // bytes per key row
  static constexpr int SLOTS = RB / 16;                       // 16-byte slots per row
  static constexpr int BYTES = kRowBlock * RB;                // one row block
  static constexpr int PER_WAVE = BYTES / 1024 / kGramWaves;  // 1 KB direct loads per wave per row block
  static constexpr int PER = PER_WAVE + 1;                    // + one norm load
  static constexpr int COUNT = kGramRingBytes / BYTES;        // ring depth: 4 (bf16), 2 (fp32)
  static_assert(kRowBlock % kGramWaves == 0 && BYTES % (1024 * kGramWaves) == 0, "row block split");
  static_assert(COUNT >= 2 && RKV_MAX_QROWS <= kRowBlock, "the query rows reuse one stage");
};

// Waits until at most `later` row blocks of PER direct-to-LDS loads each,
// issued by this wave after the awaited one, are still in flight.
template <int PER>
__device__ inline void wait_later_stages(int later) {
  static_assert(3 * PER < 64, "vmcnt has 6 bits");
  switch (later) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PER)); break;
  }
}

// Issues the direct-to-LDS loads of one 64-row block: row r of the block
// lands at st_rows + r*RB with 16-byte slot p holding the row's bytes
// [16*(p ^ (r & 15)), +16). voff[q] is the lane's block-invariant byte offset
// for load q; the block's first byte enters through the scalar offset. Rows
// past the buffer's extent read as zeros.
template <typename T>
__device__ inline void issue_rows(char* st_rows, __amdgpu_buffer_rsrc_t r, const uint32_t* voff, uint32_t soff,
                                  int wave) {
  using S = Stage<T>;
#pragma unroll
  for (int q = 0; q < S::PER_WAVE; ++q) buf_to_lds16(r, st_rows + (wave * S::PER_WAVE + q) * 1024, voff[q], soff);
}

// MFMA operand fragment of staged row R (the lane's half hh) from a swizzled stage.
template <typename T>
__device__ inline void frag_from_stage(Frag<T>& f, const char* st_rows, int R, int hh) {
  using S = Stage<T>;
  const char* row = st_rows + R * S::RB;
  const int sw = R & 15;
#pragma unroll
  for (int s = 0; s < Frag<T>::kU4; ++s) f.v[s] = *(const uint4*)(row + (((hh * (S::SLOTS / 2) + s) ^ sw) * 16));
}

// Work unit of a block id: longest units first (column group 0 of every
// slice, then group 1, ...) and, when the slices split evenly over the XCDs,
// every unit of a slice on one XCD so that its row blocks are re-read from
// that XCD's L2. Work-groups are dispatched round-robin over the XCDs and in
// id order within one.
__device__ inline void gram_unit(int bid, int slices, int& slice, int& grp) {
  if (slices % kXcds == 0) {
    const int xcd = bid % kXcds, local = bid / kXcds, per = slices / kXcds;
    grp = local / per;
    slice = xcd * per + local % per;
  } else {
    grp = bid / slices;
    slice = bid % slices;
  }
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

  __shared__ __align__(16) char rows_lds[S::COUNT * S::BYTES];
  __shared__ __align__(16) float nrm_lds[S::COUNT][kRowBlock];
  __shared__ __align__(16) float qM[RKV_MAX_QROWS];
  __shared__ __align__(16) float qInvS[RKV_MAX_QROWS];
  __shared__ __align__(16) int qPos[RKV_MAX_QROWS];
  __shared__ __align__(16) float sv[kHeadDim];

  int slice, grp, l, b, h, s0, N;
  gram_unit(blockIdx.x, g.L * g.batch * g.H, slice, grp);
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;
  if (grp * kGroupCols >= N) return;  // uniform over the block

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, col = lane & 31;
  const int jb0 = grp * kGramWaves;            // first row block of the group
  const int cbase = (jb0 + wave) * kRowBlock;  // this wave's first column = row block jb0 + wave
  const bool has_cols = cbase < N;
  const size_t srow = (size_t)slice * g.n_slots;
  const float* norms_row = norms + srow + s0;
  const int nb = gram_row_blocks(N, grp);

  // the slice's valid rows and norms as range-checked buffers
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(row_ptr<T>(k.p[l], g, b, h, s0), (uint32_t)N * RB);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(norms_row, (uint32_t)N * 4);

  // block-invariant per-lane offsets of the row-block loads
  uint32_t voff[S::PER_WAVE];
#pragma unroll
  for (int q = 0; q < S::PER_WAVE; ++q) {
    const int flat = (wave * S::PER_WAVE + q) * 64 + lane;
    const int r = flat / S::SLOTS, p = flat % S::SLOTS;
    voff[q] = (uint32_t)r * RB + (uint32_t)(p ^ (r & 15)) * 16;
  }
  constexpr int kNormsPerWave = kRowBlock / kGramWaves;
  const uint32_t nvoff = (uint32_t)(wave * kNormsPerWave + lane) * 4;
  auto issue = [&](int bi) {  // row block bi of this group into stage bi % COUNT
    const int stg = bi % S::COUNT, rbase = (jb0 + bi) * kRowBlock;
    issue_rows<T>(rows_lds + stg * S::BYTES, rk, voff, (uint32_t)rbase * RB, wave);
    if (lane < kNormsPerWave) buf_to_lds4(rn, nrm_lds[stg] + wave * kNormsPerWave, nvoff, (uint32_t)rbase * 4);
  };

  // per-slice constants of the importance and the row mean (visible after
  // the first barrier)
  if (tid < RKV_MAX_QROWS) {
    const bool row_ok = tid < g.qrows;
    qM[tid] = row_ok ? rowstat[((size_t)slice * RKV_MAX_QROWS + tid) * 2] : 0.f;
    qInvS[tid] = row_ok ? rowstat[((size_t)slice * RKV_MAX_QROWS + tid) * 2 + 1] : 0.f;
    qPos[tid] = row_ok ? N - g.alpha + tid % g.alpha : -1;  // last key the row's query attends to
  }
  if (tid < kHeadDim) sv[tid] = svec[(size_t)slice * kHeadDim + tid];
  for (int bi = 0; bi < nb && bi < S::COUNT; ++bi) issue(bi);

  // the observation queries of the slice, staged into a free ring stage for
  // the importance pass
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(
      (const char*)obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * RB, (uint32_t)g.qrows * RB);
  const int qstg = nb >= 2 ? (nb - 2) % S::COUNT : 0;

  // ---- row blocks in arrival order: MFMA, then count similar pairs
  Frag<T> bf[2];           // the wave's column keys, set at its diagonal block
  float nrm_i[2] = {0.f, 0.f}, tn[2] = {0.f, 0.f};
  uint32_t cnt[2] = {0u, 0u};
  const int i0 = cbase + col;  // column of cnt[0]; cnt[1] is column i0 + 32
  for (int bi = 0; bi < nb; ++bi) {
    // blocks issued so far: the first COUNT, then one refill per iteration
    // from iteration 1 on (block bi' - 1 + COUNT in iteration bi'), so the
    // last one issued before this wait is max(COUNT - 1, bi + COUNT - 2)
    const int last = min(nb - 1, max(S::COUNT - 1, bi + S::COUNT - 2));
    wait_later_stages<S::PER>(last - bi);
    __syncthreads();  // every wave's share of row block bi is in LDS, and every
                      // wave is done with block bi - 1, whose stage is free
    if (bi >= 1 && bi - 1 + S::COUNT < nb) issue(bi - 1 + S::COUNT);
    if (bi == nb - 1 && nb >= 2) issue_rows<T>(rows_lds + qstg * S::BYTES, rq, voff, 0u, wave);  // block nb-2's stage
    // row blocks before the wave's own columns have no pair j > i
    if (bi < wave || !has_cols) continue;
    const int stg = bi % S::COUNT;
    const char* st = rows_lds + stg * S::BYTES;
    const int rbase = (jb0 + bi) * kRowBlock;
    if (bi == wave) {  // the diagonal block holds the wave's own columns
#pragma unroll
      for (int is = 0; is < 2; ++is) {
        frag_from_stage(bf[is], st, 32 * is + col, hh);
        nrm_i[is] = nrm_lds[stg][32 * is + col];
        tn[is] = g.tau * fabsf(nrm_i[is]);  // a zero key (norm -1) compares as a unit-norm key with G = 0
      }
    }
    const bool masked = bi == wave || rbase + kRowBlock > N;  // diagonal or ragged block
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      Frag<T> af;
      frag_from_stage(af, st, 32 * js + col, hh);
      f32x16 acc0 = {}, acc1 = {};
      mma_frag(acc0, af, bf[0]);
      mma_frag(acc1, af, bf[1]);
      float nj[16];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 v = *(const float4*)&nrm_lds[stg][32 * js + 8 * a + 4 * hh];
        nj[4 * a + 0] = fabsf(v.x);
        nj[4 * a + 1] = fabsf(v.y);
        nj[4 * a + 2] = fabsf(v.z);
        nj[4 * a + 3] = fabsf(v.w);
      }
      // similar iff G_ij > tau |k_i| |k_j|, i.e. iff d = tau|k_i| |k_j| - G_ij is
      // negative: one fma per element, then its sign bit is counted (no
      // compare / carry chain)
      if (masked) {
        const int jrow0 = rbase + 32 * js;
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
  }

  // ---- both half-waves hold rows of the same columns; each column has one owner
#pragma unroll
  for (int is = 0; is < 2; ++is) {
    const uint32_t c = cnt[is] + __shfl_xor(cnt[is], 32);
    const int i = cbase + 32 * is + col;
    if (hh == 0 && i < N) counts[srow + s0 + i] = (int32_t)c;
  }

  // ---- the query rows: issued with the last block, or now when there was one block
  if (nb < 2) {
    __syncthreads();  // every wave is done with stage 0
    issue_rows<T>(rows_lds + qstg * S::BYTES, rq, voff, 0u, wave);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (!has_cols) return;
  const char* qs = rows_lds + qstg * S::BYTES;

  // ---- importance of the wave's 64 columns
  const int ntile = (g.qrows + 31) >> 5;
  const float scale = 1.0f / sqrtf((float)kHeadDim);
  const int alpha = g.alpha;
  const bool pow2 = (alpha & (alpha - 1)) == 0;
  const uint32_t magic = (65536u + (uint32_t)alpha - 1u) / (uint32_t)alpha;  // m / alpha = (m * magic) >> 16 for m < 64
#pragma unroll
  for (int is = 0; is < 2; ++is) {
    const int i = cbase + 32 * is + col;
    // attention weights of the column against every query row: lane holds
    // rows 32t + 8a + 4hh + {0..3} (a = r / 4) of tile t in register r
    float v[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t < ntile) {
        Frag<T> qf;
        frag_from_stage(qf, qs, 32 * t + col, hh);
        f32x16 acc = {};
        mma_frag(acc, qf, bf[is]);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int m0 = 32 * t + 8 * a + 4 * hh;
          const float4 vm = *(const float4*)&qM[m0];
          const float4 vs = *(const float4*)&qInvS[m0];
          const int4 vp = *(const int4*)&qPos[m0];
          const float mm[4] = {vm.x, vm.y, vm.z, vm.w}, ss[4] = {vs.x, vs.y, vs.z, vs.w};
          const int pp[4] = {vp.x, vp.y, vp.z, vp.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            // every weight is computed; the causal / validity mask multiplies it
            const float w = __expf(acc[4 * a + c] * scale - mm[c]) * ss[c];
            v[t][4 * a + c] = (i <= pp[c] && i < N) ? w : 0.f;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[t][r] = 0.f;
      }
    }
    // sum over each query's window of alpha rows, max over the GQA group
    float best = 0.f;
    if (pow2) {
      // a window is an aligned run of alpha rows: row bits 0, 1 are register
      // bits 0, 1; bit 2 is the half-wave; bits 3, 4 are register bits 2, 3;
      // bit 5 is the tile
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int sh = 1; sh <= 8; sh <<= 1) {
          const int span = sh < 4 ? sh : 2 * sh;  // rows covered by register bit log2(sh)
          if (alpha > span) {
            float u[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) u[r] = v[t][r] + v[t][r ^ sh];
#pragma unroll
            for (int r = 0; r < 16; ++r) v[t][r] = u[r];
          }
          if (sh == 2 && alpha > 4) {
#pragma unroll
            for (int r = 0; r < 16; ++r) v[t][r] += __shfl_xor(v[t][r], 32);
          }
        }
      }
      if (alpha > 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[0][r] += v[1][r];
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) best = fmaxf(best, v[t][r]);
      best = fmaxf(best, __shfl_xor(best, 32));
    } else {
      // windows not aligned to the register layout: one pass per GQA member
      const int G = g.qrows / alpha;
      for (int gq = 0; gq < G; ++gq) {
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t m = 32u * t + (uint32_t)acc_row(r, hh);
            sum += ((m * magic) >> 16) == (uint32_t)gq ? v[t][r] : 0.f;
          }
        sum += __shfl_xor(sum, 32);
        best = fmaxf(best, sum);
      }
    }
    if (hh == 0 && i < N) importance[srow + s0 + i] = best / (float)alpha;
  }

  // ---- row mean of cosine through the sum of unit keys:
  // sum_{j != i} S_ij = khat_i . s - khat_i . khat_i
  const float inv_nm1 = 1.f / (float)(N - 1);
#pragma unroll
  for (int is = 0; is < 2; ++is) {
    float dot = 0.f;
#pragma unroll
    for (int e4 = 0; e4 < 16; ++e4) {
      const float4 sd = *(const float4*)&sv[hh * 64 + 4 * e4];
      dot = fmaf(frag_val(bf[is], 4 * e4), sd.x, dot);
      dot = fmaf(frag_val(bf[is], 4 * e4 + 1), sd.y, dot);
      dot = fmaf(frag_val(bf[is], 4 * e4 + 2), sd.z, dot);
      dot = fmaf(frag_val(bf[is], 4 * e4 + 3), sd.w, dot);
    }
    dot += __shfl_xor(dot, 32);
    const int i = cbase + 32 * is + col;
    if (hh == 0 && i < N) {
      const float inv = nrm_i[is] > 0.f ? 1.f / nrm_i[is] : 0.f;
      const float self = nrm_i[is] > 0.f ? 1.f : 0.f;
      rowmean[srow + s0 + i] = (dot * inv - self) * inv_nm1;
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
