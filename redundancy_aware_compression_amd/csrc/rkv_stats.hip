// K1 — per-part statistics of one slice's keys, the bandwidth-bound first
// pass of R-KV scoring.
//
// Importance (R-KV notes page, yoonschallenge.tistory.com/1236, summary table
// row "importance computation") needs, for every observation query row
// m = g*alpha + t, the maximum and the sum of exp over the causal softmax
// row; redundancy needs key norms (Q&A part 2, cause 3: key normalisation)
// and, through the identity sum_{j != i} S_ij = khat_i . s - khat_i . khat_i,
// the sum s of unit keys. The keys are read once from HBM and the pass emits:
//   norms[slot]                      ||k_j|| in fp32 from exact bf16 values
//                                    (-1 for a zero key)
//   stats[part][m] = (max, sum exp)  of q_m . k_j / sqrt(D) over the part's keys
//   ssum[part][d]                    sum over the part's keys of k_j[d] / ||k_j||
//
// A work-group of 4 waves takes a contiguous range of 32-key blocks of one
// slice; each wave streams every 4th block through its own two-stage LDS
// ring filled by direct buffer-to-LDS loads (whole 1 KB lines per load,
// hardware range checks past the slice), so the waves never wait for each
// other until the end. Per block a wave reads its keys as MFMA A fragments
// (lane = key row half, XOR-swizzled slots), computes the logits against the
// queries held as B fragments in registers (each lane then owns one query
// row and 16 keys of the block) and keeps that row's running max and sum of
// exp; the norm and the lane's 64 dimensions of the running sum of unit keys
// are plain fp32 arithmetic on the same registers. Lanes, half-waves and
// waves are combined once, at the end.
#include "rkv_device.hpp"

namespace rkv {

constexpr int kKeyBlock = 32;  // keys per wave and block

template <typename T>
struct KeyBlock {
  static constexpr int RB = kHeadDim * Elem<T>::kBytes;  // bytes per key row
  static constexpr int SLOTS = RB / 16;                   // 16-byte slots per row
  static constexpr int BYTES = kKeyBlock * RB;            // 8 KB (bf16), 16 KB (fp32)
  static constexpr int LOADS = BYTES / 1024;              // 1 KB direct loads per block
  static constexpr int STAGES = sizeof(T) == 2 ? 4 : 2;  // ring stages per wave (128 KB per work-group)
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * 64;
};

// s_waitcnt immediates (gfx9 encoding): vmcnt(v) with the other counters
// unconstrained, and lgkmcnt(0) with the others unconstrained.
__device__ constexpr int stats_vmcnt(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkmZero = 15 | (7 << 4) | (3 << 14);

// Waits until at most nb blocks of LOADS loads and ns single stores, issued
// after the awaited block, are in flight (immediates: one case per count).
template <int LOADS, int STAGES>
__device__ inline void wait_ring(int nb, int ns) {
  static_assert((STAGES - 1) * (LOADS + 1) < 64, "vmcnt has 6 bits");
#define RKV_WAIT_CASE(B, S)                                         \
  case (B) * 4 + (S):                                               \
    __builtin_amdgcn_s_waitcnt(stats_vmcnt((B) * LOADS + (S))); \
    break;
  switch (nb * 4 + ns) {
    RKV_WAIT_CASE(0, 0) RKV_WAIT_CASE(0, 1) RKV_WAIT_CASE(0, 2) RKV_WAIT_CASE(0, 3)
    RKV_WAIT_CASE(1, 0) RKV_WAIT_CASE(1, 1) RKV_WAIT_CASE(1, 2) RKV_WAIT_CASE(1, 3)
    RKV_WAIT_CASE(2, 0) RKV_WAIT_CASE(2, 1) RKV_WAIT_CASE(2, 2) RKV_WAIT_CASE(2, 3)
    RKV_WAIT_CASE(3, 0) RKV_WAIT_CASE(3, 1) RKV_WAIT_CASE(3, 2)
    default: __builtin_amdgcn_s_waitcnt(stats_vmcnt(3 * LOADS + 3)); break;
  }
#undef RKV_WAIT_CASE
}

// 32-key blocks [lo, hi) of part `part` of a slice split `split` ways: the
// same partition for every sequence (from n_slots), clipped to its N keys.
__device__ inline void part_blocks(int n_slots, int N, int split, int part, int& lo, int& hi) {
  const int nb = (n_slots + kKeyBlock - 1) / kKeyBlock;
  const int per = (nb + split - 1) / split;
  lo = part * per;
  hi = min((N + kKeyBlock - 1) / kKeyBlock, lo + per);
}

// Merges the softmax statistics (m2, s2) into (m1, s1).
__device__ inline void merge_ms(float& m1, float& s1, float m2, float s2) {
  const float m = fmaxf(m1, m2);
  if (m == -INFINITY) return;
  s1 = (m1 > -INFINITY ? s1 * __expf(m1 - m) : 0.f) + (m2 > -INFINITY ? s2 * __expf(m2 - m) : 0.f);
  m1 = m;
}

template <typename T, int NT>  // NT query tiles of 32 rows (G * alpha <= 32 * NT)
__global__ __launch_bounds__(KeyBlock<T>::THREADS) void stats_kernel(Geom g, LayerPtrs k, const void* __restrict__ obs_q,
                                                              const int32_t* __restrict__ seq_start,
                                                              float* __restrict__ norms, float* __restrict__ stats,
                                                              float* __restrict__ ssum, float* __restrict__ rowstat,
                                                              float* __restrict__ svec, int split) {
  using KB = KeyBlock<T>;
  constexpr int RB = KB::RB;
  constexpr int kStatsWaves = KB::WAVES;
  constexpr int kStatsThreads = KB::THREADS;
  __shared__ __align__(16) char ring[kStatsWaves * KB::STAGES * KB::BYTES];
  __shared__ __align__(16) float msr[kStatsWaves * 64 * 2];  // per wave and query row: max, sum of exp
  static_assert(kStatsWaves * 64 * 64 * 4 <= kStatsWaves * KB::STAGES * KB::BYTES, "end-of-pass scratch");

  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = wid / split, part = wid % split;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;  // uniform over the block
  int lo, hi;
  part_blocks(g.n_slots, N, split, part, lo, hi);
  if (lo >= hi) return;

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to scalar registers
  const size_t srow = (size_t)slice * g.n_slots;
  // this wave's blocks: lo + wave, lo + wave + 4, ... through its own ring
  const u32x4_t rk = make_desc(row_ptr<T>(k.p[l], g, b, h, s0), (uint32_t)N * RB);
  const uint32_t my_ring = lds_addr(ring) + wave * KB::STAGES * KB::BYTES;
  uint32_t voff[KB::LOADS];
#pragma unroll
  for (int q = 0; q < KB::LOADS; ++q) {
    const int flat = q * 64 + lane;
    const int r = flat / KB::SLOTS, p = flat % KB::SLOTS;
    voff[q] = (uint32_t)r * RB + (uint32_t)(p ^ (r & 15)) * 16;
  }
  auto issue = [&](int blk, int stg) {
#pragma unroll
    for (int q = 0; q < KB::LOADS; ++q)
      dma_to_lds16(rk, my_ring + stg * KB::BYTES + q * 1024, voff[q], (uint32_t)blk * KB::BYTES);
  };
  const int nmine = hi - lo > wave ? (hi - lo - wave + kStatsWaves - 1) / kStatsWaves : 0;
  for (int i = 0; i < KB::STAGES && i < nmine; ++i) issue(lo + wave + kStatsWaves * i, i);
  // the queries as MFMA B fragments (lane: query row 32t + col, half hh);
  // rows past the group's queries are zeros. They are waited for together
  // with the first two blocks, before the loop: the compiler then knows they
  // have landed and places no wait for them inside it (a wait that would
  // also hold up the ring's loads, which it does not see)
  Frag<T> qf[NT];
  {
    const char* qbase = (const char*)obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * RB;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int m = 32 * t + col;
      if (m < g.qrows)
        frag_load(qf[t], qbase + (size_t)m * RB + hh * (RB / 2));
      else
        frag_zero(qf[t]);
    }
  }

  __builtin_amdgcn_s_waitcnt(stats_vmcnt(0));

  const float scale = 1.0f / sqrtf((float)kHeadDim);
  const int alpha = g.alpha;
  const uint32_t magic = (65536u + (uint32_t)alpha - 1u) / (uint32_t)alpha;  // m / alpha = (m * magic) >> 16 for m < 64
  float M[NT], S[NT];  // query row 32t + col over this lane's keys
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    M[t] = -INFINITY;
    S[t] = 0.f;
  }
  float run[64];  // the lane's 64 dimensions of the sum of unit keys over its keys
#pragma unroll
  for (int e = 0; e < 64; ++e) run[e] = 0.f;

  // norms go out through a range-checked buffer: lanes of the second half
  // and keys past the slice write beyond its extent and are dropped, so one
  // store instruction is issued per block whatever the lanes hold (the ring
  // waits below count it)
  const __amdgpu_buffer_rsrc_t rnorm = make_rsrc(norms + srow + s0, (uint32_t)N * 4);
  uint32_t prev_off = 0xFFFFFFF0u;
  float prev_norm = 0.f;
  for (int i = 0; i < nmine; ++i) {
    // issued after block i: the later blocks already in flight (iteration k
    // issues block k + STAGES) and one norm store per iteration since block
    // i went out (iteration k stores block k - 1's norms before its load)
    const int nb_later = min(nmine - 1, i + KB::STAGES - 1) - i;
    const int ns_later = i < KB::STAGES ? max(0, i - 1) : KB::STAGES - 1;
    wait_ring<KB::LOADS, KB::STAGES>(nb_later, ns_later);
    const int blk = lo + wave + kStatsWaves * i, stg = i % KB::STAGES;
    const char* st = ring + (wave * KB::STAGES + stg) * KB::BYTES;
    Frag<T> kf;
    {
      const char* row = st + col * RB;
      const int sw = col & 15;
#pragma unroll
      for (int s = 0; s < Frag<T>::kU4; ++s)
        kf.v[s] = *(const uint4*)(row + (((hh * (KB::SLOTS / 2) + s) ^ sw) * 16));
    }
    // the block is in registers: its stage is refilled at once, so two
    // blocks stay in flight while this one is processed (the previous
    // block's norms go out first)
    __builtin_amdgcn_s_waitcnt(kLgkmZero);
    if (i >= 1) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(prev_norm), rnorm, prev_off, 0, 0);
    if (i + KB::STAGES < nmine) issue(blk + KB::STAGES * kStatsWaves, stg);
    // norm of key j and the lane's share of the sum of unit keys
    const int j = blk * kKeyBlock + col;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      const float x = frag_val(kf, e);
      ss = fmaf(x, x, ss);
    }
    ss += __shfl_xor(ss, 32);
    const float nrm = sqrtf(ss);  // rows past the slice read as zeros
    const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
    prev_norm = nrm > 0.f ? nrm : -1.f;  // -1 marks a zero key
    prev_off = hh == 0 ? (uint32_t)j * 4u : 0xFFFFFFF0u;
    // the values are unpacked again rather than kept from the first pass
#pragma unroll
    for (int s = 0; s < Frag<T>::kU4; ++s) {
      uint32_t a = kf.v[s].x, b2 = kf.v[s].y, c = kf.v[s].z, d = kf.v[s].w;
      asm volatile("" : "+v"(a), "+v"(b2), "+v"(c), "+v"(d));
      kf.v[s] = make_uint4(a, b2, c, d);
    }
#pragma unroll
    for (int e = 0; e < 64; ++e) run[e] = fmaf(frag_val(kf, e), inv, run[e]);
    // logits: keys as rows, query rows as columns
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t] = f32x16{};
      mma_frag(acc[t], kf, qf[t]);
    }

    // running softmax statistics of the lane's query row over its 16 keys
    // of the block (registers r: keys acc_row(r, hh))
    const bool edge = blk * kKeyBlock + kKeyBlock > N - alpha;  // causal or past-the-slice keys inside
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t m = 32u * t + (uint32_t)col;
      const int pos = N - alpha + (int)(m - ((m * magic) >> 16) * (uint32_t)alpha);  // query's token
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = acc[t][r] * scale;
        if (edge) {
          const int jr = blk * kKeyBlock + acc_row(r, hh);
          x[r] = (jr < N && jr <= pos) ? x[r] : -INFINITY;
        }
        mx = fmaxf(mx, x[r]);
      }
      if (mx > -INFINITY) {
        const float Mn = fmaxf(M[t], mx);
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += __expf(x[r] - Mn);
        S[t] = (M[t] > -INFINITY ? S[t] * __expf(M[t] - Mn) : 0.f) + sum;
        M[t] = Mn;
      }
    }
  }

  if (nmine >= 1) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(prev_norm), rnorm, prev_off, 0, 0);

  // ---- combine: the two half-waves hold different keys of the same query row
#pragma unroll
  for (int t = 0; t < NT; ++t) merge_ms(M[t], S[t], __shfl_xor(M[t], 32), __shfl_xor(S[t], 32));
  __syncthreads();  // every wave is done with its ring: it becomes scratch
  float* red = (float*)ring;  // [wave][lane][64] sums of unit keys
#pragma unroll
  for (int e = 0; e < 64; ++e) red[(wave * 64 + lane) * 64 + e] = run[e];
  if (hh == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      msr[(wave * 64 + 32 * t + col) * 2] = t < NT ? M[t < NT ? t : 0] : -INFINITY;
      msr[(wave * 64 + 32 * t + col) * 2 + 1] = t < NT ? S[t < NT ? t : 0] : 0.f;
    }
  }
  __syncthreads();
  const size_t pbase = (size_t)slice * chunks_of(g.n_slots) + part;
  if (split == 1) {
    // the only part: the final statistics, (max, 1 / sum of exp) per query
    // row and (0, 0) for rows past the group's queries
    if (tid < RKV_MAX_QROWS) {
      float m1 = -INFINITY, s1 = 0.f;
#pragma unroll
      for (int w = 0; w < kStatsWaves; ++w) merge_ms(m1, s1, msr[(w * 64 + tid) * 2], msr[(w * 64 + tid) * 2 + 1]);
      rowstat[((size_t)slice * RKV_MAX_QROWS + tid) * 2] = tid < g.qrows ? m1 : 0.f;
      rowstat[((size_t)slice * RKV_MAX_QROWS + tid) * 2 + 1] = tid < g.qrows ? 1.f / s1 : 0.f;
    }
  } else if (tid < g.qrows) {
    float m1 = -INFINITY, s1 = 0.f;
#pragma unroll
    for (int w = 0; w < kStatsWaves; ++w) merge_ms(m1, s1, msr[(w * 64 + tid) * 2], msr[(w * 64 + tid) * 2 + 1]);
    stats[(pbase * RKV_MAX_QROWS + tid) * 2] = m1;
    stats[(pbase * RKV_MAX_QROWS + tid) * 2 + 1] = s1;
  }
  {
    // dimension d: half d / 64 of the rows, element d % 64; TPD threads
    // share its 32 lanes x kStatsWaves partial sums
    constexpr int TPD = kStatsThreads / kHeadDim;
    static_assert(TPD * kHeadDim == kStatsThreads && (TPD == 2 || TPD == 4), "threads per dimension");
    const int d = tid / TPD, qq = tid % TPD, half = d >> 6, e = d & 63;
    float acc_s = 0.f;
    for (int w = 0; w < kStatsWaves; ++w)
#pragma unroll
      for (int c = qq; c < 32; c += TPD) acc_s += red[(w * 64 + half * 32 + c) * 64 + e];
    acc_s += __shfl_xor(acc_s, 1);
    if (TPD == 4) acc_s += __shfl_xor(acc_s, 2);
    if (qq == 0) {
      if (split == 1)
        svec[(size_t)slice * kHeadDim + d] = acc_s;
      else
        ssum[pbase * kHeadDim + d] = acc_s;
    }
  }
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
  int nparts = 0;  // parts whose block range is non-empty (they come first)
  for (int p = 0; p < split; ++p) {
    int lo, hi;
    part_blocks(g.n_slots, N, split, p, lo, hi);
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
// one, each walking a contiguous range of blocks (long ranges amortise each
// work-group's start and its final reduction). With one per slice the pass
// writes the final statistics itself.
inline int stats_split(const Geom& g) {
  const int slices = g.L * g.batch * g.H;
  const int want = (256 + slices - 1) / slices;
  const int nch = chunks_of(g.n_slots);
  return want < 1 ? 1 : (want > nch ? nch : want);
}

int launch_reduce_stats(const Geom& g, const int32_t* seq_start, const float* stats, const float* ssum,
                        float* rowstat, float* svec, void* stream) {
  const int slices = g.L * g.batch * g.H;
  const int split = stats_split(g);
  if (slices == 0 || split == 1) return 0;  // one part per slice: the statistics pass wrote the results
  hipLaunchKernelGGL(reduce_stats_kernel, dim3(slices), dim3(256), 0, (hipStream_t)stream, g, seq_start, stats, ssum,
                     rowstat, svec, split);
  return (int)hipGetLastError();
}

int launch_stats(const Geom& g, int dtype, const LayerPtrs& k, const void* obs_q, const int32_t* seq_start,
                 float* norms, float* stats, float* ssum, float* rowstat, float* svec, void* stream) {
  const int slices = g.L * g.batch * g.H;
  const int split = stats_split(g);
  const int blocks = slices * split;
  if (blocks == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(blocks);
  if (dtype == RKV_BF16) {
    const dim3 threads(KeyBlock<bf16_t>::THREADS);
    if (g.qrows <= 32)
      hipLaunchKernelGGL((stats_kernel<bf16_t, 1>), grid, threads, 0, s, g, k, obs_q, seq_start, norms, stats, ssum,
                         rowstat, svec, split);
    else
      hipLaunchKernelGGL((stats_kernel<bf16_t, 2>), grid, threads, 0, s, g, k, obs_q, seq_start, norms, stats, ssum,
                         rowstat, svec, split);
  } else {
    const dim3 threads(KeyBlock<float>::THREADS);
    if (g.qrows <= 32)
      hipLaunchKernelGGL((stats_kernel<float, 1>), grid, threads, 0, s, g, k, obs_q, seq_start, norms, stats, ssum,
                         rowstat, svec, split);
    else
      hipLaunchKernelGGL((stats_kernel<float, 2>), grid, threads, 0, s, g, k, obs_q, seq_start, norms, stats, ssum,
                         rowstat, svec, split);
  }
  return (int)hipGetLastError();
}

}  // namespace rkv
