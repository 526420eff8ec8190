// K3 — the R-KV scoring pass: key statistics, redundancy Gram, importance
// and row mean of one slice per work-group.
//
// R-KV notes page, yoonschallenge.tistory.com/1236: summary table rows
// "importance computation" (attention of the observation queries, max over
// the GQA group) and "redundancy computation" (key cosine similarity with
// the beta most recent similar tokens protected); Q&A part 2, cause 3
// (key normalisation, all-pairs cosine). For each valid token i the pass
// needs the number of newer tokens j > i whose cosine
// S_ij = k_i.k_j / (|k_i| |k_j|) exceeds tau, the mean cosine to the other
// tokens, and the importance. The pairwise part is a dense contraction over
// head_dim = 128, run on the 32x32x16 bf16 MFMA with exact bf16 products and
// fp32 accumulation.
//
// One work-group of 8 waves per slice walks the slice's column groups in
// turn. Column group g is the 512 older tokens of row blocks 8g .. 8g+7
// (64 tokens each), wave w holding block 8g+w as MFMA B fragments in
// registers; it meets every row block of newer tokens from 8g to the end of
// the slice. All groups' row blocks form one stream through an LDS ring
// (7 stages of 16 KB) filled by direct buffer-to-LDS loads (no staging
// registers, hardware range checks past the slice). One barrier covers two
// blocks of the stream; a wave refills a stage right after its Gram work on
// a block once every wave is past the stage, so the refills spread over the
// iteration and the ring prefetches across group boundaries. LDS rows are XOR-swizzled in 16-byte slots so the MFMA operand
// reads are conflict-free. A wave has nothing to do before its own block; it
// takes its columns from the ring there (no separate column loads), so about
// the upper triangle j >= i is computed.
//
// One iteration ahead of its Gram work every block is also read by all 8
// waves for its row norms (fp32 from the exact bf16 values, 8 lanes per
// row). Group 0 meets every key of the slice, so while it streams the same
// reads give the sum of unit keys s = sum_j k_j / |k_j| and each wave takes
// one 16x16 tile (16 keys x 16 query rows) of the observation-query logits
// on the 16x16x32 MFMA, every lane keeping the running max and sum of exp of
// one query row (causal mask on the newest keys). At the end of group 0 these
// merge into the softmax statistics and s that every group's epilogue uses;
// the keys are read from HBM once.
//
// Epilogue per element of the Gram: one fma, tau*|k_i|*|k_j| - G_ij, whose
// sign bit is shifted into a per-lane mask, counted once per block. Rows
// past the slice read as zero keys with norm 0 and give +0 (for tau < 0 the
// column keys are held negated and the complement is counted, so that this
// stays true), so only the diagonal block needs the j > i mask. The N x N matrix never leaves
// registers; each column belongs to one lane, which stores its count (no
// atomics).
//
// After a group's last row block every wave computes, for its columns, the
// importance (the logits again, normalised by each query row's max and sum
// of exp, mean over the window, max over the GQA group; the window sums are
// taken in registers) and the row mean of S through
// sum_{j != i} S_ij = khat_i . s - khat_i . khat_i, while the ring already
// loads the next group's rows.
//
// The fused eviction step (FUSE) keeps the work-group on its slice after the
// last group: it selects the slice's tokens and compacts its K and V rows in
// place (fused_tail), so that each compute unit's copy phases fall between
// its scoring phases instead of all copies running after all scoring.
#include <type_traits>

#include "rkv_compact.hpp"
#include "rkv_select.hpp"
#include "rkv_tiles.hpp"

namespace rkv {

constexpr int kGramThreads = kGramWaves * 64;
static_assert(RKV_MAX_QROWS <= kRowBlock, "the query rows fill one stage-sized region");
static_assert(kRowBlock == 8 * kGramWaves, "pre-pass: 8 lanes per row, 8 rows per wave");


// bf16 keys only: fp32 keys take the scoring pass of rkv_f32.hip.
template <typename T>
struct Stage {
  static_assert(sizeof(T) == 2, "the Gram kernel takes bf16 keys");
  static constexpr int RB = kHeadDim * Elem<T>::kBytes;  // bytes per key row
  static constexpr int SLOTS = RB / 16;                   // 16-byte slots per row
  static constexpr int BYTES = kRowBlock * RB;            // one row block
  static constexpr int PER = BYTES / 1024 / kGramWaves;   // 1 KB direct loads per wave per row block
  static constexpr int COUNT = 7;                         // ring depth (LDS: ring + queries + norms <= 160 KB)
  static constexpr int NCACHE = 5120;                     // tokens whose norms stay in LDS after group 0
  static_assert(kRowBlock % kGramWaves == 0 && BYTES % (1024 * kGramWaves) == 0, "row block split");
  static_assert(COUNT >= 3 && COUNT <= 8, "ring depth");
};

// Waits until this wave's loads of the awaited row block have landed: at
// most `later` row blocks of PER direct-to-LDS loads each were issued by this
// wave after it.
template <int PER>
__device__ inline void wait_later_blocks(int later) {
  static_assert(7 * PER < 64, "vmcnt has 6 bits");
  switch (later) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PER)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * PER)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * PER)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * PER)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7 * PER)); break;
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
  for (int q = 0; q < S::PER; ++q) dma_to_lds16(r, st_rows + (wave * S::PER + q) * 1024, voff[q], soff);
}

// 16x16 logit tiles: lane l supplies row (l % 16) of a tile and, per
// 16x16x32 MFMA, 8 dims of its quarter l / 16; the result holds column
// l % 16 and rows 4 (l / 16) + r in register r.
template <typename T>
struct Tile16;
template <>
struct Tile16<bf16_t> {
  struct F {
    uint4 v[4];  // dims 32 s + 8 quarter + (0..7)
  };
  __device__ static void load(F& f, const char* st_rows, int R, int quarter) {
    const char* row = st_rows + R * (kHeadDim * 2);
    const int sw = R & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s) f.v[s] = *(const uint4*)(row + (((4 * s + quarter) ^ sw) * 16));
  }
  __device__ static void mma(f32x4& acc, const F& a, const F& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v[s]),
                                                    __builtin_bit_cast(bf16x8_t, b.v[s]), acc, 0, 0, 0);
  }
};
// 16 consecutive dims [16 c, +16) of staged row R as fp32 (exact widening).
template <typename T>
__device__ inline void row_chunk16(float* x, const char* st_rows, int R, int c) {
  using S = Stage<T>;
  constexpr int SPC = S::SLOTS / 8;  // 16-byte slots per 16 dims
  const char* row = st_rows + R * S::RB;
  const int sw = R & 15;
#pragma unroll
  for (int u = 0; u < SPC; ++u) {
    const uint4 v = *(const uint4*)(row + (((c * SPC + u) ^ sw) * 16));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[u * 8 + 2 * e] = __uint_as_float(w[e] << 16);
      x[u * 8 + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

// Sum over each aligned group of 8 lanes, in every lane of the group: two
// quad permutations, then the mirror inside the half-row (DPP, no LDS).
__device__ inline float sum8_dpp(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  return v;
}

// The rest of the eviction step for one slice, by the work-group that scored
// it (FUSE): the selection from the counts, row means and importance the
// scoring pass just wrote, then the in-place compaction of the slice's K and
// V rows, while its keys are still in the caches. The keys and the
// selection's histograms take the LDS of the row ring (`lds`). seq_start is
// left alone: other work-groups of the launch still read it (start_kernel
// writes it afterwards). With sent_id (SkipKV's sentence deduction, SkipKV
// notes page, summary table row "final eviction score") Z loses the
// sentence penalties and the sentence-id sidecar moves with the rows.
template <typename T>
__device__ inline void fused_tail(const Geom& g, int slice, int l, int b, int h, int s0, int N, const LayerPtrs& k,
                                  const LayerPtrs& v, const float* importance, const int32_t* counts,
                                  const float* rowmean, int32_t* keep, const float* sent_pen, int32_t* sent_id,
                                  int s_max, char* lds) {
  constexpr int RB = kHeadDim * Elem<T>::kBytes;
  constexpr size_t KEYS = (size_t)RKV_MAX_CAPACITY * 4;
  // every store of this work-group's scoring is complete before any wave reads
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (sent_id)  // (uniform)
    select_slice<true, true>(g, slice, b, s0, N, importance, nullptr, counts, rowmean, keep, nullptr, nullptr,
                             sent_pen, sent_id, s_max, (uint32_t*)lds, *(SelectLds*)(lds + KEYS));
  else
    select_slice<true, false>(g, slice, b, s0, N, importance, nullptr, counts, rowmean, keep, nullptr, nullptr,
                              nullptr, nullptr, 0, (uint32_t*)lds, *(SelectLds*)(lds + KEYS));
  __builtin_amdgcn_s_waitcnt(0);  // the keep row is written before it is read
  __syncthreads();
  const int32_t* krow = keep + (size_t)slice * g.budget;
  const size_t off = ((size_t)b * g.H + h) * g.capacity * (size_t)RB;
  compact_rows<T>((char*)k.p[l] + off, krow, g);
  compact_rows<T>((char*)v.p[l] + off, krow, g);
  if (sent_id) {  // ids[j] <- ids[keep[j]], -1 where keep[j] < 0: every read staged in LDS before any write
    int32_t* irow = sent_id + (size_t)slice * g.capacity;
    int32_t* stage = (int32_t*)lds;  // the selection's keys are no longer needed
    for (int j = threadIdx.x; j < g.budget; j += blockDim.x) {
      const int kj = krow[j];
      stage[j] = (kj >= 0 && kj < g.n_slots) ? irow[kj] : -1;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < g.budget; j += blockDim.x) irow[j] = stage[j];
  }
}

// A sequence's first valid slot after the fused step, from the keep row of
// its (layer 0, KV head 0) slice.
__global__ void start_kernel(Geom g, const int32_t* __restrict__ keep, int32_t* __restrict__ seq_start) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < g.batch) seq_start[b] = leading_unkept(keep + (size_t)b * g.H * g.budget, g.budget);
}

// GATHER: the slice's valid tokens are virtual slots [s0, n_slots); virtual
// slot v < budget is stored at physical slot order[v], v >= budget at v (the
// layout the hole-filling compaction keeps). The row loads gather physical
// rows in virtual order; everything else works in virtual slots.
// CAPT: the importance comes from the attention weights that decode steps
// captured, imp_acc [slices][G][capacity] (sums over the observation window):
// I = max over the group of the sum / alpha. The queries are not read and the
// logit work is left out; only with GATHER = false.
// FUSE: the work-group goes on to the slice's selection and compaction
// (fused_tail; only with GATHER = false; v and keep are used only then).
template <typename T, bool GATHER, bool CAPT, bool FUSE>
__global__ __launch_bounds__(kGramThreads) void gram_kernel(Geom g, LayerPtrs k, LayerPtrs v,
                                                            const void* __restrict__ obs_q,
                                                            const int32_t* __restrict__ seq_start,
                                                            const int32_t* __restrict__ order,
                                                            const float* __restrict__ imp_acc,
                                                            float* __restrict__ importance,
                                                            float* __restrict__ rowmean, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ keep,
                                                            const float* __restrict__ sent_pen,
                                                            int32_t* __restrict__ sent_id, int s_max) {
  static_assert(!(GATHER && CAPT), "captured importance is indexed by virtual slot only without GATHER");
  static_assert(!(GATHER && FUSE), "the fused step keeps the order-preserving layout");
  using S = Stage<T>;
  using TL = Tile16<T>;
  constexpr int RB = S::RB;

  __shared__ __align__(16) char rows_lds[S::COUNT * S::BYTES];
  __shared__ __align__(16) char q_lds[S::BYTES];               // the slice's query rows
  __shared__ __align__(16) float nrm_lds[S::COUNT][kRowBlock];  // row norms per stage (-1: zero key, 0: past the slice)
  __shared__ __align__(16) float nrm_all[S::NCACHE];            // the same per token, kept from group 0 on
  __shared__ __align__(16) float rst_lds[RKV_MAX_QROWS * 2];   // per query row: max, 1 / sum of exp
  __shared__ __align__(16) float sv_lds[kHeadDim];             // sum of unit keys
  __shared__ __align__(16) char s_lds[32 * RB];                // s as MFMA rows; scratch before that
  constexpr int KA = 4;  // GATHER: refills between an ORD load and its use
  __shared__ __align__(16) int ord_lds[GATHER ? KA : 1][kGramWaves][8];  // GATHER: order entries of a wave's rows
  static_assert(kGramWaves * (2 * 16 * 2 + kHeadDim) * 4 <= 32 * RB, "merge scratch fits the s tile");
  static_assert((size_t)RKV_MAX_CAPACITY * 4 + sizeof(SelectLds) <= sizeof(rows_lds), "the fused tail's LDS");
  static_assert(kGramThreads == kSelectThreads && kGramThreads == kCompactThreads, "one work-group size");

  const int slice = xcd_remap(blockIdx.x, gridDim.x);
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) {
    if constexpr (FUSE) fused_tail<T>(g, slice, l, b, h, s0, N, k, v, importance, counts, rowmean, keep, sent_pen, sent_id,
                                            s_max, rows_lds);
    return;
  }

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to scalar registers
  const size_t srow = (size_t)slice * g.n_slots;
  const int ngroups = gram_groups(N);
  const int nrb = (N + kRowBlock - 1) / kRowBlock;  // row blocks of the slice
  // every group's row blocks in one stream: group gg contributes nrb - 8 gg
  const int total = ngroups * nrb - kGroupBlocks * ngroups * (ngroups - 1) / 2;

  // the slice's valid rows (GATHER: all its physical rows below n_slots) as a
  // range-checked buffer
  const u32x4_t rk = GATHER ? make_desc(row_ptr<T>(k.p[l], g, b, h, 0), (uint32_t)g.n_slots * RB)
                            : make_desc(row_ptr<T>(k.p[l], g, b, h, s0), (uint32_t)N * RB);
  const uint32_t ring = lds_addr(rows_lds);

  // block-invariant per-lane offsets of the row-block loads: load q of a
  // wave brings row r = 8 wave + (64 q + lane) / SLOTS of the block, bytes
  // 16 (p ^ (r & 15)) .. of it (vpart)
  static_assert(S::PER * 64 / S::SLOTS * kGramWaves == kRowBlock, "each wave loads 8 whole rows");
  constexpr int KPQ = 64 / S::SLOTS;  // rows per load
  uint32_t voff[S::PER];
#pragma unroll
  for (int q = 0; q < S::PER; ++q) {
    const int flat = (wave * S::PER + q) * 64 + lane;
    const int r = flat / S::SLOTS, p = flat % S::SLOTS;
    voff[q] = (uint32_t)r * RB + (uint32_t)(p ^ (r & 15)) * 16;
  }
  // the in-row part of load q's offset (row 8 wave + KPQ q + lane / SLOTS)
  auto vpart = [&](int q) { return voff[q] - (uint32_t)(8 * wave + KPQ * q + lane / S::SLOTS) * RB; };

  // ---- loads: the first row block, the queries (all waves), the rest of
  // the ring; the issue cursor walks the stream (block ibi of group ig)
  int ig = 0, ibi = 0;
  auto cursor_step = [&]() {
    if (++ibi == nrb - ig * kGroupBlocks) {
      ++ig;
      ibi = 0;
    }
  };
  const int pro_n = min(total, S::COUNT);  // blocks issued before the loop
  // GATHER: the physical slots of a block's rows come from the order table.
  // The prologue reads them with ordinary loads (for its blocks and for the
  // first refill's), awaited before the first direct-to-LDS load. Later
  // blocks' slots come through LDS: ORD(X), a direct-to-LDS load of the 8
  // entries of each wave's rows, is issued two refills ahead, and read into
  // registers (noff) at the end of the refill before X; ORD(X) is issued
  // KA refills ahead, so that waiting for it needs no younger row block than
  // the ring already waits for. Each wave's sequence of vector memory
  // operations is therefore ORD(COUNT + 1) .. ORD(COUNT + KA - 1) (those
  // before the stream's end), ROW(0), the queries, ROW(1) .. ROW(pro_n - 1),
  // then per refill of block X: ORD(X + KA) (when X + KA < total) and ROW(X);
  // end_row(X) counts the operations up to ROW(X), so every wait is exact.
  const int o0 = GATHER ? max(0, min(KA - 1, total - S::COUNT - 1)) : 0;
  auto end_row = [&](int X) -> int {
    if (X == 0) return o0 + S::PER;
    if (X < S::COUNT) return o0 + (X + 2) * S::PER;
    const int nord = GATHER ? max(0, min(X, total - KA - 1) - S::COUNT + 1) : 0;
    return o0 + (pro_n + 1) * S::PER + (X - S::COUNT + 1) * S::PER + nord;
  };
  // operations up to ORD(Y), Y > COUNT
  auto end_ord = [&](int Y) -> int { return Y < S::COUNT + KA ? Y - S::COUNT : end_row(Y - KA) - S::PER; };
  const int32_t* ord = GATHER ? order + (size_t)slice * g.budget : nullptr;
  auto phys_of = [&](int v, int o) { return v < g.budget ? o : (v < g.n_slots ? v : g.n_slots); };
  const u32x4_t odesc = GATHER ? make_desc(ord, (uint32_t)g.budget * 4u) : rk;
  // virtual slot of row 0 of stream block X (uniform)
  auto vbase_of = [&](int X) {
    int gg = 0;
    while (X >= nrb - gg * kGroupBlocks) X -= nrb - (gg++) * kGroupBlocks;
    return s0 + (gg * kGroupBlocks + X) * kRowBlock;
  };
  // ORD(X): the order entries of the wave's 8 rows of block X (lanes 0..7)
  auto issue_ord = [&](int X) {
    if (lane < 8)
      dma_to_lds4(odesc, lds_addr(&ord_lds[X % KA][wave][0]),
                  (uint32_t)min(vbase_of(X) + 8 * wave + lane, g.budget - 1) * 4u, 0u);
  };
  auto issue_row = [&](int q, const uint32_t* off, int rbase) {
    if constexpr (GATHER)
      issue_rows<T>(ring + (q % S::COUNT) * S::BYTES, rk, off, 0u, wave);
    else
      issue_rows<T>(ring + (q % S::COUNT) * S::BYTES, rk, voff, (uint32_t)rbase * RB, wave);
  };
  uint32_t noff[S::PER];  // GATHER: the load offsets of the next refill's block
  // a refill: block X = the cursor's block
  auto issue_next = [&](int X) {
    const int rbase = (ig * kGroupBlocks + ibi) * kRowBlock;
    cursor_step();
    if (GATHER && X + KA < total) issue_ord(X + KA);
    issue_row(X, noff, rbase);
    if (GATHER && X + 1 < total) {
      wait_vm(end_row(X) - end_ord(X + 1));
      asm volatile("" ::: "memory");  // the LDS reads below follow that wait
      const int vb = s0 + (ig * kGroupBlocks + ibi) * kRowBlock + 8 * wave;
#pragma unroll
      for (int qq = 0; qq < S::PER; ++qq) {
        const int kk = KPQ * qq + lane / S::SLOTS;
        noff[qq] = (uint32_t)phys_of(vb + kk, ord_lds[(X + 1) % KA][wave][kk]) * RB + vpart(qq);
      }
    }
  };
  {
    // the prologue's blocks and the first refill's
    uint32_t poff[S::COUNT + 1][S::PER];
    if constexpr (GATHER) {
      int cg = 0, cb = 0;
#pragma unroll
      for (int X = 0; X <= S::COUNT; ++X) {
#pragma unroll
        for (int qq = 0; qq < S::PER; ++qq) {
          const int v = s0 + (cg * kGroupBlocks + cb) * kRowBlock + 8 * wave + KPQ * qq + lane / S::SLOTS;
          // (unconditional: a block past the stream gets an unused, in-range read)
          poff[X][qq] = (uint32_t)phys_of(v, ord[min(v, g.budget - 1)]) * RB + vpart(qq);
        }
        if (++cb == nrb - cg * kGroupBlocks) {
          ++cg;
          cb = 0;
        }
      }
      // all loads issued above; every value is awaited here, before any
      // direct-to-LDS load
#pragma unroll
      for (int X = 0; X <= S::COUNT; ++X)
#pragma unroll
        for (int qq = 0; qq < S::PER; ++qq) asm volatile("" : "+v"(poff[X][qq]));
#pragma unroll
      for (int qq = 0; qq < S::PER; ++qq) noff[qq] = poff[S::COUNT][qq];
      for (int Y = S::COUNT + 1; Y < S::COUNT + 1 + o0; ++Y) issue_ord(Y);
    }
    issue_row(0, poff[0], 0);
    cursor_step();
    // (the queries come before ROW(1), so no wait on a later block counts them)
    if constexpr (!CAPT)
      issue_rows<T>(lds_addr(q_lds),
                    make_desc((const char*)obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * RB,
                              (uint32_t)g.qrows * RB),
                    voff, 0u, wave);
#pragma unroll
    for (int X = 1; X < S::COUNT; ++X) {
      if (X < pro_n) {
        issue_row(X, poff[X], (ig * kGroupBlocks + ibi) * kRowBlock);
        cursor_step();
      }
    }
  }

  const float scale = 1.0f / sqrtf((float)kHeadDim);
  // tau < 0: the wave holds its column keys negated and counts the newer
  // tokens with S_ij < tau (tau*|k_i||k_j| - G_ij > 0 becomes a sign test on
  // |tau||k_i||k_j| + G_ij), then takes the complement over the valid newer
  // tokens. Rows past the slice (zero keys, norm 0) then give +0 and never
  // count, whatever the sign of tau. The epilogue's products with the
  // column keys change sign with them (csgn).
  const bool negtau = g.tau < 0.f;
  const float csgn = negtau ? -1.f : 1.f;
  const float escale = csgn * scale;
  const int alpha = g.alpha;
  const bool pow2 = (alpha & (alpha - 1)) == 0;
  const uint32_t magic = (65536u + (uint32_t)alpha - 1u) / (uint32_t)alpha;  // m / alpha = (m * magic) >> 16 for m < 64
  const int ntile = (g.qrows + 31) >> 5;
  const int nqt16 = (g.qrows + 15) >> 4;  // 16-row query tiles of the logit tiles
  const float inv_nm1 = 1.f / (float)(N - 1);

  // ---- pre-pass state: the lane's row in the block (8 lanes per row) and
  // its 16 dims; in group 0 also its share of s and its logit tiles
  const int pr = 8 * wave + (lane >> 3), pc = lane & 7;
  float run[16];  // s over the lane's rows, dims 16 pc + (0..15)
#pragma unroll
  for (int e = 0; e < 16; ++e) run[e] = 0.f;
  float tM[2] = {-INFINITY, -INFINITY}, tS[2] = {0.f, 0.f};  // logit tiles wave and wave + 8
  int pg = 0, pbi = 0;  // the pre-pass cursor: block pbi of group pg
  // row block blk keeps its norms in nrm_all once group 0 has seen it
  auto cached = [&](int blk) { return (blk + 1) * kRowBlock <= S::NCACHE; };
  // norms of stream block q, and with FIRST (a group-0 block) the statistics
  auto pre = [&](int q, auto first) {
    constexpr bool FIRST = decltype(first)::value;
    const int stg = q % S::COUNT;
    const char* st = rows_lds + stg * S::BYTES;
    const int blk = pg * kGroupBlocks + pbi;  // row block of the slice
    if (++pbi == nrb - pg * kGroupBlocks) {
      ++pg;
      pbi = 0;
    }
    if (!FIRST && cached(blk)) return;  // its norms are in LDS since group 0
    float x[16];
    row_chunk16<T>(x, st, pr, pc);
    float ss4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
#pragma unroll
    for (int e = 0; e < 16; ++e) ss4[e & 3] = fmaf(x[e], x[e], ss4[e & 3]);
    const float nrm = sqrtf(sum8_dpp((ss4[0] + ss4[1]) + (ss4[2] + ss4[3])));  // the row's 8 lanes
    const int j = blk * kRowBlock + pr;  // token of the row
    const float nv = j < N ? (nrm > 0.f ? nrm : -1.f) : 0.f;
    if (pc == 0) {
      nrm_lds[stg][pr] = nv;
      if (FIRST && cached(blk)) nrm_all[j] = nv;
    }
    if constexpr (FIRST) {
      const float inv = nrm > 0.f ? __builtin_amdgcn_rcpf(nrm) : 0.f;  // rows past the slice are zeros
#pragma unroll
      for (int e = 0; e < 16; ++e) run[e] = fmaf(x[e], inv, run[e]);
      // logit tiles t = wave, wave + 8: keys 16 (t % 4) .. of the block,
      // query rows 16 (t / 4) ..; lane: query row (lane & 15), keys 4 (lane >> 4) + r
      if constexpr (CAPT) return;
      const bool edge = blk * kRowBlock + kRowBlock > N - alpha;  // causal or past-the-slice keys inside
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = wave + 8 * u;
        if (t >= 4 * nqt16) break;
        const int kt = t & 3, qt = t >> 2;
        typename TL::F ka;
        TL::load(ka, st, 16 * kt + (lane & 15), lane >> 4);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        typename TL::F qf;  // the query rows' fragment, read from LDS (fewer live registers than keeping it)
        TL::load(qf, q_lds, 16 * qt + (lane & 15), lane >> 4);
        TL::mma(acc, ka, qf);
        const uint32_t m = 16u * qt + (uint32_t)(lane & 15);
        const int pos = N - alpha + (int)(m - ((m * magic) >> 16) * (uint32_t)alpha);  // query's token
        float xs[4], mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xs[r] = acc[r] * scale;
          if (edge) {
            const int jr = blk * kRowBlock + 16 * kt + 4 * (lane >> 4) + r;
            xs[r] = (jr < N && jr <= pos) ? xs[r] : -INFINITY;
          }
          mx = fmaxf(mx, xs[r]);
        }
        if (mx > -INFINITY) {
          const float Mn = fmaxf(tM[u], mx);
          float sum = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) sum += __expf(xs[r] - Mn);
          tS[u] = (tM[u] > -INFINITY ? tS[u] * __expf(tM[u] - Mn) : 0.f) + sum;
          tM[u] = Mn;
        }
      }
    }
  };

  using First = std::integral_constant<bool, true>;
  using Later = std::integral_constant<bool, false>;

  // Stream blocks per barrier: the pre-pass runs BPB blocks ahead of the
  // Gram work, so one barrier covers BPB blocks (their norms written by other
  // waves, the next BPB blocks landed, the stages of the previous BPB free).
  // The ring holds BPB blocks in Gram work, BPB in the pre-pass and at least
  // BPB in flight. (The gathered stream's order-table loads are counted per
  // refill, in the refills' order, which the pairs do not change.)
  constexpr int BPB = 2;
  static_assert(S::COUNT >= 3 * BPB, "ring depth for the blocks per barrier");
  auto pre_any = [&](int x) {
    if (x < nrb)
      pre(x, First{});
    else
      pre(x, Later{});
  };

  // blocks 0 .. BPB - 1 and the queries (issued after ROW(0), before ROW(1))
  if constexpr (GATHER)
    wait_vm(pro_n == 1 ? 0 : end_row(pro_n - 1) - max(end_row(min(BPB, pro_n) - 1), o0 + 2 * S::PER));
  else
    wait_later_blocks<S::PER>(pro_n - min(BPB, pro_n));
  __syncthreads();
#pragma unroll 1
  for (int x = 0; x < BPB && x < total; ++x) pre_any(x);

  Frag<T> bf[2];  // this group's column keys of the wave: fragment f holds columns cbase + 32 f + (0..31)
  float tn[2] = {0.f, 0.f}, nrm_i[2] = {0.f, 0.f};
  uint32_t cnt[2] = {0u, 0u};

  // the start of stream iteration q (a multiple of BPB): blocks q + BPB ..
  // q + 2 BPB - 1 must have landed for their pre-pass. Blocks issued so far:
  // the first COUNT, then one refill per block (BPB = 1: block q' - 1 + COUNT
  // at iteration q' >= 1, after its barrier; BPB = 2: block q' - 2 + COUNT
  // after Gram block q' >= 2), the last before this wait being
  // max(COUNT - 1, q - 1 - BPB + COUNT)
  auto advance = [&](int q) {
    if (q + BPB < total) {
      const int last = min(total - 1, max(S::COUNT - 1, q - 1 - BPB + S::COUNT));
      const int need = min(total - 1, q + 2 * BPB - 1);
      if constexpr (GATHER)
        wait_vm(end_row(last) - end_row(need));
      else
        wait_later_blocks<S::PER>(last - need);
    }
    __syncthreads();  // the norms of blocks q .. q + BPB - 1 are in LDS, the
                      // next BPB blocks have landed, and every wave is done
                      // with blocks q - BPB .. q - 1, whose stages are free
    if (BPB == 1) {
      const int X = q - 1 + S::COUNT;
      if (X >= S::COUNT && X < total) issue_next(X);
    }
  };
  // BPB = 2: after Gram block q, the refill of the stage of block q - 2
  // (every wave passed the barrier at the start of q's iteration after
  // finishing q - 2), issued here rather than all at the barrier so that the
  // waves' loads do not queue up together
  auto refill2 = [&](int q) {
    const int X = q - 2 + S::COUNT;
    if (BPB == 2 && X >= S::COUNT && X < total) issue_next(X);
  };

  // Gram work of stream block q = block bi of group gg
  auto gram_block = [&](int q, int gg, int bi) {
    const int cbase = (gg * kGroupBlocks + wave) * kRowBlock;  // the wave's columns in this group
    if (bi >= wave && cbase < N) {  // row blocks before the wave's own have no pair j > i
      const int stg = q % S::COUNT;
      const char* st = rows_lds + stg * S::BYTES;
      const int blk = gg * kGroupBlocks + bi;
      const float* ns = cached(blk) ? nrm_all + blk * kRowBlock : nrm_lds[stg];
      const bool diag = bi == wave;
      if (diag) {  // the block's rows are the wave's columns
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          frag_from_stage(bf[f], st, 32 * f + col, hh);
          if (negtau) frag_negate(bf[f]);
          nrm_i[f] = ns[32 * f + col];
          tn[f] = fabsf(g.tau) * fabsf(nrm_i[f]);  // a zero key (norm -1) compares as G = 0
        }
      }
      uint32_t bits[2] = {0u, 0u};  // sign bits of the block's 32 rows per column fragment
      if (__builtin_expect(!diag, 1)) {
        // Both 32-row halves' products first, then the first half's epilogue
        // placed between the second half's 16 MFMAs (4 VALU after each): the
        // epilogue runs in the matrix units' shadow. (With GATHER the extra
        // accumulators take the last registers and the compiler spills 16
        // bytes; spill traffic only adds vector memory operations younger
        // than the rows a wait is for, and loads return in order, so every
        // computed vmcnt wait stays sufficient.)
        float nj0[16], nj1[16];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float4 v0 = *(const float4*)&ns[8 * a + 4 * hh];
          const float4 v1 = *(const float4*)&ns[32 + 8 * a + 4 * hh];
          nj0[4 * a + 0] = fabsf(v0.x);
          nj0[4 * a + 1] = fabsf(v0.y);
          nj0[4 * a + 2] = fabsf(v0.z);
          nj0[4 * a + 3] = fabsf(v0.w);
          nj1[4 * a + 0] = fabsf(v1.x);
          nj1[4 * a + 1] = fabsf(v1.y);
          nj1[4 * a + 2] = fabsf(v1.z);
          nj1[4 * a + 3] = fabsf(v1.w);
        }
        Frag<T> af0, af1;
        frag_from_stage(af0, st, col, hh);
        frag_from_stage(af1, st, 32 + col, hh);
        f32x16 a00 = {}, a01 = {}, a10 = {}, a11 = {};
        mma_frag(a00, af0, bf[0]);
        mma_frag(a01, af0, bf[1]);
        mma_frag(a10, af1, bf[0]);
        mma_frag(a11, af1, bf[1]);
        bits[0] = sign_bits(a00, tn[0], nj0, 0u);
        bits[1] = sign_bits(a01, tn[1], nj0, 0u);
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // the first half's MFMAs
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one of the second half's
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four epilogue VALU
        }
        bits[0] = sign_bits(a10, tn[0], nj1, bits[0]);
        bits[1] = sign_bits(a11, tn[1], nj1, bits[1]);
      } else
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

  };

  // end of group 0: every key of the slice went through the pre-pass
  auto merge_stats = [&]() {
    // Lanes 16 apart hold the same query row (other keys); lanes 8 apart
    // the same dims (other rows).
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (CAPT) break;
      merge_ms(tM[u], tS[u], lane_xor16(tM[u]), lane_xor16(tS[u]));
      merge_ms(tM[u], tS[u], lane_xor32(tM[u]), lane_xor32(tS[u]));
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      run[e] = xor8_add(run[e]);
      run[e] = xor16_add(run[e]);
      run[e] = xor32_add(run[e]);
    }
    float* msc = (float*)s_lds;                  // [wave][tile u][16 rows][2]
    float* usc = msc + kGramWaves * 2 * 16 * 2;  // [wave][128 dims]
    if (lane < 16) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        msc[((wave * 2 + u) * 16 + lane) * 2] = tM[u];
        msc[((wave * 2 + u) * 16 + lane) * 2 + 1] = tS[u];
      }
    }
    if (lane < 8) {
#pragma unroll
      for (int e = 0; e < 16; ++e) usc[wave * kHeadDim + 16 * lane + e] = run[e];
    }
    __syncthreads();
    // query row m: tiles t = 4 (m / 16) + kt, kt = 0..3, held by wave t % 8 in slot t / 8
    float Mf = -INFINITY, Sf = 0.f, sd = 0.f;
    if (!CAPT && tid < RKV_MAX_QROWS) {
      const int qt = tid >> 4;
      if (qt < nqt16) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int t = 4 * qt + kt;
          const int base = (((t & 7) * 2 + (t >> 3)) * 16 + (tid & 15)) * 2;
          merge_ms(Mf, Sf, msc[base], msc[base + 1]);
        }
      }
    }
    if (tid < kHeadDim) {
#pragma unroll
      for (int w = 0; w < kGramWaves; ++w) sd += usc[w * kHeadDim + tid];
    }
    __syncthreads();  // the scratch is read: the tile of s rows replaces it
    if (!CAPT && tid < RKV_MAX_QROWS) {
      // rows past the group's queries get (0, 0): their weights vanish
      rst_lds[2 * tid] = tid < g.qrows ? Mf : 0.f;
      rst_lds[2 * tid + 1] = tid < g.qrows ? 1.f / Sf : 0.f;
    }
    for (int o = SRows<T>::ROWS * RB + tid * 16; o < 32 * RB; o += kGramThreads * 16)
      *(uint4*)(s_lds + o) = make_uint4(0, 0, 0, 0);
    if (tid < kHeadDim) {
      sv_lds[tid] = sd;
      SRows<T>::write(s_lds, tid, sd);
    }
    __syncthreads();
  };

  // after a group's last block: counts, row mean and importance of the
  // wave's columns (the ring keeps loading the next group's rows)
  auto epilogue = [&](int gg) {
    const int cbase = (gg * kGroupBlocks + wave) * kRowBlock;
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
          const uint32_t c = xor32_add(cnt[f]);  // both half-waves hold rows of the column
          if (hh == 0 && i < N) {
            const float dot = csgn * SRows<T>::dot(accs[f]);
            counts[srow + s0 + i] = negtau ? (int32_t)(N - 1 - i) - (int32_t)c : (int32_t)c;
            const float inv = nrm_i[f] > 0.f ? 1.f / nrm_i[f] : 0.f;
            const float self = nrm_i[f] > 0.f ? 1.f : 0.f;
            rowmean[srow + s0 + i] = (dot * inv - self) * inv_nm1;
          }
        }
      }
      if constexpr (CAPT) {
        // the captured sums of the window's weights: max over the group, / alpha
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int i = cbase + 32 * f + col;
          if (hh == 0 && i < N) {
            const float* a = imp_acc + (size_t)slice * g.G * g.capacity + s0 + i;
            float best = a[0];
            for (int gq = 1; gq < g.G; ++gq) best = fmaxf(best, a[(size_t)gq * g.capacity]);
            importance[srow + s0 + i] = best / (float)alpha;
          }
        }
        cnt[0] = cnt[1] = 0u;
        return;
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
            for (int c = 0; c < 4; ++c) v[4 * a + c] = __expf(acc[4 * a + c] * escale - mm[c]) * ss[c];
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
                for (int r = 0; r < 16; ++r) v[r] = xor32_add(v[r]);
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
              sum = xor32_add(sum);
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
          best = xor32_max(best);
        }
        if (hh == 0 && i < N) importance[srow + s0 + i] = best / (float)alpha;
      }
    }
    cnt[0] = cnt[1] = 0u;
  };

  // The stream: group 0 (with the statistics pre-pass over every key of the
  // slice), then the later groups; after a group's last block its epilogue
  // (after group 0 the statistics merge first). The barrier and the pre-pass
  // come every BPB blocks; a pair of blocks may straddle a group's end.
  auto step = [&](int q, auto first) {
    if (q % BPB == 0) {
      advance(q);
#pragma unroll 1
      for (int x = q + BPB; x < q + 2 * BPB && x < total; ++x) {
        if constexpr (decltype(first)::value)
          pre_any(x);
        else
          pre(x, Later{});
      }
    }
  };
  for (int q = 0; q < nrb; ++q) {
    step(q, First{});
    gram_block(q, 0, q);
    refill2(q);
  }
  merge_stats();
  epilogue(0);
  // the later groups
  int q = nrb;
  for (int gg = 1; gg < ngroups; ++gg) {
    const int nbg = nrb - gg * kGroupBlocks;  // row blocks of this group
    for (int bi = 0; bi < nbg; ++bi, ++q) {
      step(q, Later{});
      gram_block(q, gg, bi);
      refill2(q);
    }
    epilogue(gg);
  }
  if constexpr (FUSE) fused_tail<T>(g, slice, l, b, h, s0, N, k, v, importance, counts, rowmean, keep, sent_pen, sent_id,
                                            s_max, rows_lds);
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
                const int32_t* order, float* importance, float* rowmean, int32_t* counts, void* stream,
                const float* imp_acc) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  if (order && imp_acc) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(slices), block(kGramThreads);
#define RKV_GRAM(T, GA, CA)                                                                                   \
  RKV_LAUNCH((gram_kernel<T, GA, CA, false>), grid, block, 0, s, g, k, k, obs_q, seq_start, order, imp_acc, \
                     importance, rowmean, counts, (int32_t*)nullptr, (const float*)nullptr, (int32_t*)nullptr, 0)
  if (dtype != RKV_BF16) return (int)hipErrorInvalidValue;  // fp32 keys: launch_score_f32
  if (order)
    RKV_GRAM(bf16_t, true, false);
  else if (imp_acc)
    RKV_GRAM(bf16_t, false, true);
  else
    RKV_GRAM(bf16_t, false, false);
#undef RKV_GRAM
  return 0;
}

int launch_fused_step(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const void* obs_q,
                      int32_t* seq_start, float* importance, float* rowmean, int32_t* counts, int32_t* keep,
                      void* stream, const float* imp_acc, const float* sent_pen, int32_t* sent_id, int s_max) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  if (dtype != RKV_BF16 || g.capacity > RKV_MAX_CAPACITY) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(slices), block(kGramThreads);
  if (imp_acc)
    RKV_LAUNCH((gram_kernel<bf16_t, false, true, true>), grid, block, 0, s, g, k, v, obs_q,
                       (const int32_t*)seq_start, (const int32_t*)nullptr, imp_acc, importance, rowmean, counts,
                       keep, sent_pen, sent_id, s_max);
  else
    RKV_LAUNCH((gram_kernel<bf16_t, false, false, true>), grid, block, 0, s, g, k, v, obs_q,
                       (const int32_t*)seq_start, (const int32_t*)nullptr, imp_acc, importance, rowmean, counts,
                       keep, sent_pen, sent_id, s_max);
  RKV_LAUNCH(start_kernel, dim3((g.batch + 255) / 256), dim3(256), 0, s, g, (const int32_t*)keep, seq_start);
  return 0;
}

int launch_redundancy(const Geom& g, const int32_t* seq_start, const int32_t* counts, const float* rowmean,
                      float* redundancy, void* stream) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0 || g.n_slots == 0) return 0;
  dim3 grid((g.n_slots + 255) / 256, slices);
  RKV_LAUNCH(redundancy_kernel, grid, dim3(256), 0, (hipStream_t)stream, g, seq_start, counts, rowmean,
                     redundancy);
  return 0;
}

}  // namespace rkv
