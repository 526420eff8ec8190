// K3 — redundancy Gram kernel with fused importance and row mean.
//
// Redundancy (R-KV notes page, yoonschallenge.tistory.com/1236, summary table
// row "redundancy computation"; Q&A part 2, cause 3: all-pairs key cosine)
// needs, for each valid token i, the number of newer tokens j > i whose
// cosine S_ij = k_i.k_j / (|k_i| |k_j|) exceeds tau (the protection test for
// the beta most recent similar tokens) and the mean cosine to the other
// tokens. The pairwise part is a dense contraction over head_dim = 128, run
// on the 32x32x16 bf16 MFMA with exact bf16 products and fp32 accumulation.
//
// One work-group of 8 waves per slice walks the slice's column groups in
// turn. Column group g is the 512 older tokens of row blocks 8g .. 8g+7
// (64 tokens each), wave w holding block 8g+w as MFMA B fragments in
// registers; it meets every row block of newer tokens from 8g to the end of
// the slice. All groups' row blocks form one stream through an LDS ring
// (8 stages of 16 KB) filled by direct buffer-to-LDS loads (no staging
// registers, hardware range checks past the slice); a stage is refilled as
// soon as every wave is past it, so the ring prefetches across group
// boundaries. LDS rows are XOR-swizzled in 16-byte slots so the MFMA operand
// reads are conflict-free. A wave has nothing to do before its own block; it
// takes its columns from the ring there (no separate column loads), so about
// the upper triangle j >= i is computed.
//
// Epilogue per element: one fma, tau*|k_i|*|k_j| - G_ij, whose sign bit (the
// norms come from the statistics pass) is added to the count of column i in
// the lane that owns it. Rows past the slice read as zero keys with zero
// norm and give +0, so only the diagonal block needs the j > i mask. The
// N x N matrix never leaves registers; each column belongs to one lane,
// which stores its count (no atomics).
//
// After a group's last row block every wave computes, for its columns, the
// importance (observation-query attention normalised by each query row's max
// and sum of exp from the statistics pass, mean over the window, max over
// the GQA group; the window sums are taken in registers) and the row mean of
// S through sum_{j != i} S_ij = khat_i . s - khat_i . khat_i with s the sum
// of unit keys, while the ring already loads the next group's rows. The
// queries and the per-slice constants are loaded into LDS once, first.
#include "rkv_device.hpp"

namespace rkv {

constexpr int kGramThreads = kGramWaves * 64;
static_assert(RKV_MAX_QROWS <= kRowBlock, "the query rows fill one stage-sized region");

// s_waitcnt immediate for vmcnt(v), other counters unconstrained (gfx9 encoding).
__device__ constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

template <typename T>
struct Stage {
  static constexpr int RB = kHeadDim * Elem<T>::kBytes;      // bytes per key row
  static constexpr int SLOTS = RB / 16;                       // 16-byte slots per row
  static constexpr int BYTES = kRowBlock * RB;                // one row block
  static constexpr int PER_WAVE = BYTES / 1024 / kGramWaves;  // 1 KB direct loads per wave per row block
  static constexpr int PER = PER_WAVE + 1;                    // + one norm load
  static constexpr int COUNT = sizeof(T) == 2 ? 8 : 3;        // ring depth (LDS: ring + queries <= 160 KB)
  static_assert(kRowBlock % kGramWaves == 0 && BYTES % (1024 * kGramWaves) == 0, "row block split");
  static_assert(COUNT >= 2 && COUNT <= 8, "ring depth");
};

// Waits until this wave's loads of the awaited row block have landed: at
// most `later` row blocks of PER direct-to-LDS loads each, plus EXTRA other
// loads, were issued by this wave after it.
template <int PER, int EXTRA>
__device__ inline void wait_later_blocks(int later) {
  static_assert(7 * PER + EXTRA < 64, "vmcnt has 6 bits");
  switch (later) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(EXTRA)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER + EXTRA)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER + EXTRA)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PER + EXTRA)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * PER + EXTRA)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * PER + EXTRA)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * PER + EXTRA)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7 * PER + EXTRA)); break;
  }
}

// Issues this wave's share of the direct-to-LDS loads of one 64-row block:
// row r of the block lands at st_rows + r*RB with 16-byte slot p holding the
// row's bytes [16*(p ^ (r & 15)), +16). voff[q] is the lane's block-invariant
// byte offset for load q; the block's first byte enters through the scalar
// offset. Rows past the buffer's extent read as zeros.
template <typename T>
__device__ inline void issue_rows(uint32_t st_rows, u32x4_t r, const uint32_t* voff, uint32_t soff, int wave) {
  using S = Stage<T>;
#pragma unroll
  for (int q = 0; q < S::PER_WAVE; ++q) dma_to_lds16(r, st_rows + (wave * S::PER_WAVE + q) * 1024, voff[q], soff);
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

// Similar pairs of one 32x32 tile: d = tau|k_i| |k_j| - G_ij is negative iff
// S_ij > tau; each sign bit is shifted into a per-lane mask (one alignbit per
// element, no compare / carry chain), whose bits are counted once per block.
__device__ inline uint32_t sign_bits(const f32x16& acc, float tn, const float* nj, uint32_t mask) {
#pragma unroll
  for (int r = 0; r < 16; ++r) mask = __builtin_amdgcn_alignbit(mask, __float_as_uint(fmaf(tn, nj[r], -acc[r])), 31);
  return mask;
}
// The same on the diagonal tile: only pairs whose row (newer token, index
// jl0 + acc_row within the block) lies after the column (index il).
__device__ inline uint32_t count_tile_masked(const f32x16& acc, float tn, const float* nj, int jl0, int il, int hh) {
  uint32_t c = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t sb = __float_as_uint(fmaf(tn, nj[r], -acc[r])) >> 31;
    c += jl0 + acc_row(r, hh) > il ? sb : 0u;
  }
  return c;
}

// The sum of unit keys s as MFMA rows of the key type: for bf16 three rows
// s_hi + s_mid + s_lo (each the round-to-nearest-even bf16 of what the
// previous rows leave, so the rows sum to s within 2^-27 |s|), for fp32 s
// itself. Element d of row r lives at the swizzled slot of a staged row.
__device__ inline uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
template <typename T>
struct SRows;
template <>
struct SRows<bf16_t> {
  static constexpr int RB = kHeadDim * 2;
  __device__ static void write(char* tile, int d, float s) {
    float rest = s;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const uint32_t h = f32_to_bf16_rne(rest);
      rest -= __uint_as_float(h << 16);
      const int byte = d * 2;
      *(uint16_t*)(tile + r * RB + (((byte >> 4) ^ r) << 4) + (byte & 15)) = (uint16_t)h;
    }
  }
  __device__ static float dot(const f32x16& acc) { return (acc[0] + acc[1]) + acc[2]; }
};
template <>
struct SRows<float> {
  static constexpr int RB = kHeadDim * 4;
  __device__ static void write(char* tile, int d, float s) {
    const int byte = d * 4;
    *(float*)(tile + ((byte >> 4) << 4) + (byte & 15)) = s;  // row 0: no swizzle
  }
  __device__ static float dot(const f32x16& acc) { return acc[0]; }
};
template <typename T>
__device__ inline void write_s_rows(char* tile, int d, float s) {
  SRows<T>::write(tile, d, s);
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
  __shared__ __align__(16) char q_lds[S::BYTES];               // the slice's query rows
  __shared__ __align__(16) float nrm_lds[S::COUNT][kRowBlock];
  __shared__ __align__(16) float rst_lds[RKV_MAX_QROWS * 2];  // per query row: max, 1 / sum of exp
  __shared__ __align__(16) float sv_lds[kHeadDim];            // sum of unit keys
  __shared__ __align__(16) char s_lds[32 * RB];                // s as MFMA rows (see below), swizzled

  const int slice = xcd_remap(blockIdx.x, gridDim.x);
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to scalar registers
  const size_t srow = (size_t)slice * g.n_slots;
  const float* norms_row = norms + srow + s0;
  const int ngroups = gram_groups(N);
  const int nrb = (N + kRowBlock - 1) / kRowBlock;  // row blocks of the slice
  // every group's row blocks in one stream: group gg contributes nrb - 8 gg
  const int total = ngroups * nrb - kGroupBlocks * ngroups * (ngroups - 1) / 2;

  // the slice's valid rows and norms as range-checked buffers
  const u32x4_t rk = make_desc(row_ptr<T>(k.p[l], g, b, h, s0), (uint32_t)N * RB);
  const u32x4_t rn = make_desc(norms_row, (uint32_t)N * 4);
  const uint32_t ring = lds_addr(rows_lds), nring = lds_addr(&nrm_lds[0][0]);

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

  // the tile of s rows starts as zeros: only its first rows get values
  for (int o = tid * 16; o < 32 * RB; o += kGramThreads * 16) *(uint4*)(s_lds + o) = make_uint4(0, 0, 0, 0);

  // ---- loaded first: the per-slice constants (wave 0, 512 bytes each),
  // the first row block, the queries (all waves), then the rest of the ring;
  // the first ring wait covers them all
  if (wave == 0 && lane < 32) {
    dma_to_lds16(make_desc(rowstat + (size_t)slice * RKV_MAX_QROWS * 2, RKV_MAX_QROWS * 8), lds_addr(rst_lds),
                 (uint32_t)lane * 16, 0u);
    dma_to_lds16(make_desc(svec + (size_t)slice * kHeadDim, kHeadDim * 4), lds_addr(sv_lds), (uint32_t)lane * 16,
                 0u);
  }
  // the issue cursor walks the stream: block ibi of group ig
  int ig = 0, ibi = 0;
  auto issue_next = [&](int q) {  // stream block q (the cursor's block) into stage q % COUNT
    const int stg = q % S::COUNT, rbase = (ig * kGroupBlocks + ibi) * kRowBlock;
    issue_rows<T>(ring + stg * S::BYTES, rk, voff, (uint32_t)rbase * RB, wave);
    if (lane < kNormsPerWave)
      dma_to_lds4(rn, nring + (stg * kRowBlock + wave * kNormsPerWave) * 4, nvoff, (uint32_t)rbase * 4);
    if (++ibi == nrb - ig * kGroupBlocks) {
      ++ig;
      ibi = 0;
    }
  };
  issue_next(0);
  issue_rows<T>(lds_addr(q_lds),
                make_desc((const char*)obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * RB,
                          (uint32_t)g.qrows * RB),
                voff, 0u, wave);
  for (int q = 1; q < total && q < S::COUNT; ++q) issue_next(q);

  const float scale = 1.0f / sqrtf((float)kHeadDim);
  const int alpha = g.alpha;
  const bool pow2 = (alpha & (alpha - 1)) == 0;
  const uint32_t magic = (65536u + (uint32_t)alpha - 1u) / (uint32_t)alpha;  // m / alpha = (m * magic) >> 16 for m < 64
  const int ntile = (g.qrows + 31) >> 5;
  const float inv_nm1 = 1.f / (float)(N - 1);

  Frag<T> bf[2];  // this group's column keys of the wave: fragment f holds columns cbase + 32 f + (0..31)
  float tn[2] = {0.f, 0.f}, nrm_i[2] = {0.f, 0.f};
  uint32_t cnt[2] = {0u, 0u};
  int gg = 0, bi = 0;  // the block being processed: block bi of group gg
  for (int q = 0; q < total; ++q) {
    // blocks issued so far: the first COUNT, then one refill per iteration
    // from iteration 1 on (block q' - 1 + COUNT in iteration q'), so the last
    // one issued before this wait is max(COUNT - 1, q + COUNT - 2)
    const int last = min(total - 1, max(S::COUNT - 1, q + S::COUNT - 2));
    if (q == 0)
      wait_later_blocks<S::PER, S::PER_WAVE>(last);  // the queries went out after block 0
    else
      wait_later_blocks<S::PER, 0>(last - q);
    __syncthreads();  // every wave's share of block q is in LDS, and every
                      // wave is done with block q - 1, whose stage is free
    if (q >= 1 && q - 1 + S::COUNT < total) issue_next(q - 1 + S::COUNT);
    if (q == 0 && tid < kHeadDim) write_s_rows<T>(s_lds, tid, sv_lds[tid]);  // read after the next barrier

    const int cbase = (gg * kGroupBlocks + wave) * kRowBlock;  // the wave's columns in this group
    const int nbg = nrb - gg * kGroupBlocks;                    // row blocks of this group
    if (bi >= wave && cbase < N) {  // row blocks before the wave's own have no pair j > i
      const int stg = q % S::COUNT;
      const char* st = rows_lds + stg * S::BYTES;
      const float* ns = nrm_lds[stg];
      const bool diag = bi == wave;
      if (diag) {  // the block's rows are the wave's columns
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          frag_from_stage(bf[f], st, 32 * f + col, hh);
          nrm_i[f] = ns[32 * f + col];
          tn[f] = g.tau * fabsf(nrm_i[f]);  // a zero key (norm -1) compares as G = 0
        }
      }
      uint32_t bits[2] = {0u, 0u};  // sign bits of the block's 32 rows per column fragment
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        Frag<T> af;
        frag_from_stage(af, st, 32 * js + col, hh);
        float nj[16];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float4 v = *(const float4*)&ns[32 * js + 8 * a + 4 * hh];
          nj[4 * a + 0] = fabsf(v.x);
          nj[4 * a + 1] = fabsf(v.y);
          nj[4 * a + 2] = fabsf(v.z);
          nj[4 * a + 3] = fabsf(v.w);
        }
        f32x16 acc0 = {}, acc1 = {};
        mma_frag(acc0, af, bf[0]);
        mma_frag(acc1, af, bf[1]);
        if (__builtin_expect(!diag, 1)) {
          bits[0] = sign_bits(acc0, tn[0], nj, bits[0]);
          bits[1] = sign_bits(acc1, tn[1], nj, bits[1]);
        } else {
          cnt[0] += count_tile_masked(acc0, tn[0], nj, 32 * js, col, hh);
          cnt[1] += count_tile_masked(acc1, tn[1], nj, 32 * js, 32 + col, hh);
        }
      }
      cnt[0] += __builtin_popcount(bits[0]);
      cnt[1] += __builtin_popcount(bits[1]);
    }

    if (bi + 1 < nbg) {
      ++bi;
      continue;
    }
    // ---- the group's last block: counts, row mean and importance of the
    // wave's columns (the ring keeps loading the next group's rows)
    if (q == 0) __syncthreads();  // the s rows written in this iteration
    if (cbase < N) {
      // row mean of cosine through the sum of unit keys:
      // sum_{j != i} S_ij = khat_i . s - khat_i . khat_i, k_i . s being the sum
      // of the MFMA rows against the tile of s (registers 0.. of half 0)
      {
        Frag<T> sf;
        frag_from_stage(sf, s_lds, col, hh);
        f32x16 accs[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          accs[f] = f32x16{};
          mma_frag(accs[f], sf, bf[f]);
        }
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int i = cbase + 32 * f + col;
          const uint32_t c = cnt[f] + __shfl_xor(cnt[f], 32);  // both half-waves hold rows of the column
          if (hh == 0 && i < N) {
            const float dot = SRows<T>::dot(accs[f]);
            counts[srow + s0 + i] = (int32_t)c;
            const float inv = nrm_i[f] > 0.f ? 1.f / nrm_i[f] : 0.f;
            const float self = nrm_i[f] > 0.f ? 1.f : 0.f;
            rowmean[srow + s0 + i] = (dot * inv - self) * inv_nm1;
          }
        }
      }
      // both column fragments against the first query tile
      f32x16 accq0[2];
      {
        Frag<T> qf;
        frag_from_stage(qf, q_lds, col, hh);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          accq0[f] = f32x16{};
          mma_frag(accq0[f], qf, bf[f]);
        }
      }
      // importance: only columns among the newest alpha tokens can lie after
      // a query's position
      const bool causal_free = cbase + kRowBlock <= N - alpha;
      const int G = g.qrows / alpha;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int i = cbase + 32 * f + col;
        float best = 0.f, tsum = 0.f, carry = 0.f;
        int carry_g = -1;  // GQA member whose window continues from the previous tile
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (t >= ntile) break;
          f32x16 acc = accq0[f];
          if (t > 0) {  // the second query tile (more than 32 query rows)
            Frag<T> qf;
            frag_from_stage(qf, q_lds, 32 + col, hh);
            acc = f32x16{};
            mma_frag(acc, qf, bf[f]);
          }
          // attention weights of the column against the tile's query rows: the
          // lane holds rows 32t + 8a + 4hh + {0..3} (a = r / 4) in register r;
          // rows past the group's queries have zero queries and statistics (0, 0)
          float v[16];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int m0 = 32 * t + 8 * a + 4 * hh;
            const float4 s01 = *(const float4*)&rst_lds[2 * m0];
            const float4 s23 = *(const float4*)&rst_lds[2 * m0 + 4];
            const float mm[4] = {s01.x, s01.z, s23.x, s23.z}, ss[4] = {s01.y, s01.w, s23.y, s23.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) v[4 * a + c] = __expf(acc[4 * a + c] * scale - mm[c]) * ss[c];
            if (!causal_free) {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const uint32_t m = (uint32_t)(m0 + c);
                const int pos = N - alpha + (int)(m - ((m * magic) >> 16) * (uint32_t)alpha);  // query's token
                v[4 * a + c] = (i <= pos && i < N) ? v[4 * a + c] : 0.f;
              }
            }
          }
          // sum over each query's window of alpha rows, max over the GQA group
          if (pow2) {
            // a window is an aligned run of alpha rows: row bits 0, 1 are
            // register bits 0, 1; bit 2 is the half-wave; bits 3, 4 are
            // register bits 2, 3; bit 5 is the tile
#pragma unroll
            for (int sh = 1; sh <= 8; sh <<= 1) {
              const int span = sh < 4 ? sh : 2 * sh;  // rows covered by register bit log2(sh)
              if (alpha > span) {
                float u[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) u[r] = v[r] + v[r ^ sh];
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] = u[r];
              }
              if (sh == 2 && alpha > 4) {
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] += __shfl_xor(v[r], 32);
              }
            }
            if (alpha > 32) {
              tsum += v[0];  // a window spans both tiles
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) best = fmaxf(best, v[r]);
            }
          } else {
            // windows not aligned to the register layout: one pass per GQA
            // member with rows in this tile; at most one member's window
            // continues into the next tile
            const int g_lo = (32 * t) / alpha, g_hi = min(G - 1, (32 * t + 31) / alpha);
            for (int gq = g_lo; gq <= g_hi; ++gq) {
              float sum = 0.f;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const uint32_t m = 32u * t + (uint32_t)acc_row(r, hh);
                sum += ((m * magic) >> 16) == (uint32_t)gq ? v[r] : 0.f;
              }
              sum += __shfl_xor(sum, 32);
              if (gq == carry_g) sum += carry;
              if ((gq + 1) * alpha > 32 * (t + 1)) {
                carry = sum;
                carry_g = gq;
              } else {
                best = fmaxf(best, sum);
              }
            }
          }
        }
        if (pow2) {
          if (alpha > 32) best = tsum;
          best = fmaxf(best, __shfl_xor(best, 32));
        }
        if (hh == 0 && i < N) importance[srow + s0 + i] = best / (float)alpha;
      }
    }
    cnt[0] = cnt[1] = 0u;
    ++gg;
    bi = 0;
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
  if (slices == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == RKV_BF16)
    hipLaunchKernelGGL(gram_kernel<bf16_t>, dim3(slices), dim3(kGramThreads), 0, s, g, k, obs_q, seq_start, norms,
                       rowstat, svec, importance, rowmean, counts);
  else
    hipLaunchKernelGGL(gram_kernel<float>, dim3(slices), dim3(kGramThreads), 0, s, g, k, obs_q, seq_start, norms,
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
