// The R-KV scoring pass for fp32 keys, spread over many work-groups.
//
// R-KV notes page, yoonschallenge.tistory.com/1236: summary table rows
// "importance computation" (attention of the observation queries, max over
// the GQA group) and "redundancy computation" (key cosine similarity with
// the beta most recent similar tokens protected); Q&A part 2, cause 3 (key
// normalisation, the all-pairs cosine of every compression round). The
// outputs are those of the bf16 scoring kernel (rkv_gram.hip): per valid
// token i of an evicting slice the number of newer tokens j > i whose cosine
// S_ij exceeds tau, the mean cosine to the other tokens, and the importance.
//
// fp32 matrix products run at 1/16 of the bf16 rate on MI355X (64 flops per
// cycle and SIMD), so one work-group per slice would keep one compute unit
// busy for tens of microseconds even on a 384-token slice. The pass is cut
// three ways instead:
//   f32_stats_kernel  one work-group per chunk of 32 keys: key norms, the
//                     chunk's sum of unit keys and, per observation-query
//                     row, the (max, sum of exp) of its causal logits;
//   f32_pair_kernel   one work-group per 32x32 tile of the upper triangle
//                     (column tokens i, row tokens j >= i): each wave takes a
//                     quarter of the dims on the 32x32x2 fp32 MFMA, the
//                     quarters are summed in order, and the tile's similar
//                     pairs j > i go to the column's count with an integer
//                     atomic (the total does not depend on the order);
//   f32_final_kernel  four threads per token: row mean through the sum of unit
//                     keys, sum_{j != i} S_ij = khat_i . s - khat_i . khat_i,
//                     and importance from the logits normalised by the merged
//                     statistics (chunks merged in a fixed order).
// A zero key has cosine 0 with every key (its norm enters the threshold as
// 1, its Gram entries are 0).
#include "rkv_tiles.hpp"

namespace rkv {

constexpr int kF32Threads = 256;

// Physical slot of virtual slot v (GATHER: the hole-filling layout's order
// table for v < budget), clamped into the slice's rows.
template <bool GATHER>
__device__ inline int f32_phys(const Geom& g, const int32_t* ord, int v) {
  if constexpr (GATHER) {
    if (v < g.budget) {
      const int o = ord[v];
      return o < 0 ? 0 : (o >= g.n_slots ? g.n_slots - 1 : o);
    }
  }
  return v;
}

__device__ inline const float* f32_row(const LayerPtrs& k, const Geom& g, int l, int b, int h, int phys) {
  return (const float*)row_ptr<float>(k.p[l], g, b, h, phys);
}

// Sum over each 16-lane row of the wave, in every lane of the row (DPP).
__device__ inline float f32_row16_sum(float v) {
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1, 0, 3, 2]
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2, 3, 0, 1]
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// The slice's query rows into LDS as [QR][128] floats, rows past qrows
// zero; every load of a thread is issued before any store.
template <int QR>
__device__ inline void f32_stage_queries(float* q_lds, const float* qb, int qrows, int tid) {
  constexpr int PER = (QR * kHeadDim / 4 + kF32Threads - 1) / kF32Threads;  // float4 per thread
  float4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = (u * kF32Threads + tid) * 4;
    v[u] = e < qrows * kHeadDim ? *(const float4*)&qb[e] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = (u * kF32Threads + tid) * 4;
    if (e < QR * kHeadDim) *(float4*)&q_lds[e] = v[u];
  }
}

// Sum over each quad of lanes, in every lane of the quad (DPP).
__device__ inline float f32_quad_sum(float v) {
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0xB1, 0xF, 0xF, false));  // quad_perm [1, 0, 3, 2]
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x4E, 0xF, 0xF, false));  // quad_perm [2, 3, 0, 1]
  return v;
}

// Online (max, sum of exp) of one query row.
__device__ inline void f32_online(float& M, float& S, float x) {
  if (x > M) {
    S = (M > -INFINITY ? S * expf(M - x) : 0.f) + 1.f;
    M = x;
  } else {
    S += expf(x - M);
  }
}

// Chunk c of a slice: local tokens [32 c, 32 c + 32) of its N valid ones.
// Each 16-lane row of a wave takes one token per round (lane: dims
// [8 q, 8 q + 8), q = lane % 16); a round covers 16 tokens.
template <bool GATHER, bool CAPT, int QR>
__global__ __launch_bounds__(kF32Threads) void f32_stats_kernel(Geom g, LayerPtrs k, const float* __restrict__ obs_q,
                                                                 const int32_t* __restrict__ seq_start,
                                                                 const int32_t* __restrict__ order,
                                                                 float* __restrict__ norms, float* __restrict__ parts,
                                                                 int32_t* __restrict__ counts) {
  __shared__ __align__(16) float q_lds[CAPT ? 4 : QR * kHeadDim];
  __shared__ float red_s[kF32Threads / 64][kHeadDim];
  __shared__ float red_m[kF32Threads / 64][RKV_MAX_QROWS][2];
  const int slice = blockIdx.y, chunk = blockIdx.x;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;
  const int j0 = chunk * kF32Chunk;
  if (j0 >= N) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q16 = lane & 15, grp = lane >> 4;
  const size_t srow = (size_t)slice * g.n_slots;
  const int32_t* ord = GATHER ? order + (size_t)slice * g.budget : nullptr;
  const float scale = 1.f / sqrtf((float)kHeadDim);
  if constexpr (!CAPT) {
    f32_stage_queries<QR>(q_lds, obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * kHeadDim, g.qrows,
                          tid);
    __syncthreads();
  }
  float sacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sacc[e] = 0.f;
  float Mx[4], Sx[4];  // statistics of query rows q16 + 16 u
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    Mx[u] = -INFINITY;
    Sx[u] = 0.f;
  }
  // the lane's part of round it's row (zeros past the slice); the next
  // round's row is loaded while this one is used
  constexpr int kRounds = kF32Chunk / 16;
  auto load_round = [&](int it, float4& a, float4& c) {
    const int jl = j0 + it * 16 + wave * 4 + grp;
    if (jl < N) {
      const float4* row = (const float4*)(f32_row(k, g, l, b, h, f32_phys<GATHER>(g, ord, s0 + jl)) + 8 * q16);
      a = row[0];
      c = row[1];
    } else {
      a = c = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  float4 ca, cc, na, nc;
  load_round(0, ca, cc);
#pragma unroll 1
  for (int it = 0; it < kRounds; ++it) {
    if (it + 1 < kRounds) load_round(it + 1, na, nc);
    const int jl = j0 + it * 16 + wave * 4 + grp;  // local token of the lane's row
    const bool valid = jl < N;
    const float x[8] = {ca.x, ca.y, ca.z, ca.w, cc.x, cc.y, cc.z, cc.w};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    const float nrm = sqrtf(f32_row16_sum(ss));
    if (valid && q16 == 0) {
      norms[srow + s0 + jl] = nrm;
      counts[srow + s0 + jl] = 0;  // the pair kernel adds to it
    }
    const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sacc[e] = fmaf(x[e], inv, sacc[e]);
    if constexpr (!CAPT) {
      // per group u of 16 query rows: their logits of the row (independent
      // chains), then the lane's statistics slot u (query row q16 + 16 u)
      constexpr int GW = QR < 16 ? QR : 16;
#pragma unroll
      for (int u = 0; u < (QR + 15) / 16; ++u) {
        float lgs[GW];
#pragma unroll
        for (int c = 0; c < GW; ++c) {
          const int m = 16 * u + c;
          const float4 qa = *(const float4*)&q_lds[m * kHeadDim + 8 * q16];
          const float4 qc = *(const float4*)&q_lds[m * kHeadDim + 8 * q16 + 4];
          float d = x[0] * qa.x;
          d = fmaf(x[1], qa.y, d);
          d = fmaf(x[2], qa.z, d);
          d = fmaf(x[3], qa.w, d);
          d = fmaf(x[4], qc.x, d);
          d = fmaf(x[5], qc.y, d);
          d = fmaf(x[6], qc.z, d);
          d = fmaf(x[7], qc.w, d);
          lgs[c] = f32_row16_sum(d) * scale;
        }
        float lg = lgs[0];
#pragma unroll
        for (int c = 1; c < GW; ++c) lg = q16 == c ? lgs[c] : lg;
        const int m = q16 + 16 * u;
        const int pos = N - g.alpha + m % g.alpha;  // the query's token
        if (valid && m < g.qrows && q16 < QR && jl <= pos) f32_online(Mx[u], Sx[u], lg);
        __builtin_amdgcn_sched_barrier(0);  // one group's reads at a time (register pressure)
      }
    }
    ca = na;
    cc = nc;
  }
  // the wave's four token rows, then the waves in order
#pragma unroll
  for (int e = 0; e < 8; ++e) sacc[e] = xor32_add(xor16_add(sacc[e]));
  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red_s[wave][8 * q16 + e] = sacc[e];
  }
  if constexpr (!CAPT) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      merge_ms(Mx[u], Sx[u], lane_xor16(Mx[u]), lane_xor16(Sx[u]));
      merge_ms(Mx[u], Sx[u], lane_xor32(Mx[u]), lane_xor32(Sx[u]));
      if (grp == 0) {
        red_m[wave][q16 + 16 * u][0] = Mx[u];
        red_m[wave][q16 + 16 * u][1] = Sx[u];
      }
    }
  }
  __syncthreads();
  float* pb = parts + ((size_t)slice * f32_chunks(g.n_slots) + chunk) * kF32PartFloats;
  if (tid < kHeadDim) {
    float sv = 0.f;
#pragma unroll
    for (int w = 0; w < kF32Threads / 64; ++w) sv += red_s[w][tid];
    pb[tid] = sv;
  }
  if (!CAPT && tid < g.qrows) {
    float M = -INFINITY, S = 0.f;
#pragma unroll
    for (int w = 0; w < kF32Threads / 64; ++w) merge_ms(M, S, red_m[w][tid][0], red_m[w][tid][1]);
    pb[kHeadDim + 2 * tid] = M;
    pb[kHeadDim + 2 * tid + 1] = S;
  }
}

// Tiles of a slice with nf 32-token fragments: t = rj (rj + 1) / 2 + ci for
// column fragment ci <= row fragment rj.
__host__ __device__ inline int f32_tiles(int n) {
  const int nf = (n + 31) / 32;
  return nf * (nf + 1) / 2;
}

// One work-group per tile t of a slice. Wave w multiplies dims {16 w + d,
// 64 + 16 w + d : d < 16} (lane half hh supplies the second set) on 16
// MFMAs; the four partial tiles meet in LDS and wave 0 adds them in wave
// order, then counts.
template <bool GATHER>
__global__ __launch_bounds__(kF32Threads) void f32_pair_kernel(Geom g, LayerPtrs k, const int32_t* __restrict__ seq_start,
                                                                const int32_t* __restrict__ order,
                                                                const float* __restrict__ norms,
                                                                int32_t* __restrict__ counts) {
  __shared__ __align__(16) float part[kF32Threads / 64 - 1][16][64];  // waves 1.. : register r of lane l
  const int slice = blockIdx.y;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;
  const int t = blockIdx.x;
  if (t >= f32_tiles(N)) return;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int rj = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while ((rj + 1) * (rj + 2) / 2 <= t) ++rj;
  while (rj * (rj + 1) / 2 > t) --rj;
  const int ci = t - rj * (rj + 1) / 2;
  const size_t srow = (size_t)slice * g.n_slots;
  const int32_t* ord = GATHER ? order + (size_t)slice * g.budget : nullptr;
  const int i = 32 * ci + col;   // the lane's column token
  const int jr = 32 * rj + col;  // the row token whose operand the lane supplies
  const int d0 = 64 * hh + 16 * wave;
  uint4 a[4], c4[4];
  if (i < N) {
    const uint4* p = (const uint4*)(f32_row(k, g, l, b, h, f32_phys<GATHER>(g, ord, s0 + i)) + d0);
#pragma unroll
    for (int s = 0; s < 4; ++s) c4[s] = p[s];
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) c4[s] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (jr < N) {
    const uint4* p = (const uint4*)(f32_row(k, g, l, b, h, f32_phys<GATHER>(g, ord, s0 + jr)) + d0);
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = p[s];
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = make_uint4(0u, 0u, 0u, 0u);
  }
  float nj[16], ni = 1.f;
  if (wave == 0) {  // the norms, loaded with the operands (zero keys enter as 1)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * rj + acc_row(r, hh);
      nj[r] = j < N ? norms[srow + s0 + j] : 1.f;
    }
    ni = i < N ? norms[srow + s0 + i] : 1.f;
  }
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float* x = (const float*)&a[s];
    const float* y = (const float*)&c4[s];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x[e], y[e], acc, 0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kF32Threads / 64 - 1; ++w)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += part[w][r][lane];
  // S_ij > tau iff tau |k_i| |k_j| - G_ij < 0 (zero keys: norm 1, G = 0)
  const float tn = g.tau * (ni > 0.f ? ni : 1.f);
  uint32_t c = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = 32 * rj + acc_row(r, hh);
    if (i < N && j < N && j > i) c += fmaf(tn, nj[r] > 0.f ? nj[r] : 1.f, -acc[r]) < 0.f ? 1u : 0u;
  }
  c += lane_xor32(c);  // the two half-waves hold different rows of the column
  if (hh == 0 && i < N && c) atomicAdd(&counts[srow + s0 + i], (int)c);
}

// Four threads per token (a quad of lanes, dims [32 p, 32 p + 32) each):
// row mean and importance. QR: query rows held per thread (g.qrows rounded
// up to 8, 16, 32 or 64); rows past g.qrows have zero queries and
// statistics (0, 0), so their weights vanish.
constexpr int kF32FinalTok = kF32Threads / 4;  // tokens per work-group
template <bool GATHER, bool CAPT, int QR>
__global__ __launch_bounds__(kF32Threads) void f32_final_kernel(Geom g, LayerPtrs k, const float* __restrict__ obs_q,
                                                                 const int32_t* __restrict__ seq_start,
                                                                 const int32_t* __restrict__ order,
                                                                 const float* __restrict__ norms,
                                                                 const float* __restrict__ parts,
                                                                 const float* __restrict__ imp_acc,
                                                                 float* __restrict__ importance,
                                                                 float* __restrict__ rowmean) {
  __shared__ __align__(16) float q_lds[CAPT ? 4 : QR * kHeadDim];
  __shared__ __align__(16) float s_lds[kHeadDim];
  __shared__ float st_lds[CAPT ? 1 : QR][2];  // per query row: max, 1 / sum of exp
  const int slice = blockIdx.y;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  if (N <= g.budget) return;
  const int i0 = blockIdx.x * kF32FinalTok;
  if (i0 >= N) return;
  const int tid = threadIdx.x;
  const size_t srow = (size_t)slice * g.n_slots;
  const int32_t* ord = GATHER ? order + (size_t)slice * g.budget : nullptr;
  const float* pb = parts + (size_t)slice * f32_chunks(g.n_slots) * kF32PartFloats;
  const int nck = f32_chunks(N);
  if (tid < kHeadDim) {
    float sv = 0.f;
    for (int c0 = 0; c0 < nck; c0 += 8) {  // chunks in order, eight loads in flight at a time
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c0 + u < nck ? pb[(size_t)(c0 + u) * kF32PartFloats + tid] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) sv += v[u];
    }
    s_lds[tid] = sv;
  }
  if constexpr (!CAPT) {
    if (tid < QR) {
      float M = -INFINITY, S = 0.f;
      if (tid < g.qrows) {
        // chunks in order, eight loads in flight at a time
        for (int c0 = 0; c0 < nck; c0 += 8) {
          float2 ms[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            ms[u] = c0 + u < nck ? *(const float2*)&pb[(size_t)(c0 + u) * kF32PartFloats + kHeadDim + 2 * tid]
                                 : make_float2(-INFINITY, 0.f);
#pragma unroll
          for (int u = 0; u < 8; ++u) merge_ms(M, S, ms[u].x, ms[u].y);
        }
      }
      st_lds[tid][0] = tid < g.qrows ? M : 0.f;
      st_lds[tid][1] = tid < g.qrows ? 1.f / S : 0.f;
    }
    f32_stage_queries<QR>(q_lds, obs_q + ((size_t)(l * g.batch + b) * g.H + h) * (size_t)g.qrows * kHeadDim, g.qrows,
                          tid);
  }
  __syncthreads();
  const int i = i0 + tid / 4, qp = tid & 3;
  float ds = 0.f;
  float lg[CAPT ? 1 : QR];
#pragma unroll
  for (int m = 0; m < (CAPT ? 1 : QR); ++m) lg[m] = 0.f;
  if (i < N) {
    const float4* row = (const float4*)f32_row(k, g, l, b, h, f32_phys<GATHER>(g, ord, s0 + i)) + 8 * qp;
    float4 x4[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x4[u] = row[u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c4 = 8 * qp + u;
      const float4 x = x4[u];
      const float4 sv = *(const float4*)&s_lds[4 * c4];
      ds = fmaf(x.x, sv.x, ds);
      ds = fmaf(x.y, sv.y, ds);
      ds = fmaf(x.z, sv.z, ds);
      ds = fmaf(x.w, sv.w, ds);
      if constexpr (!CAPT) {
#pragma unroll
        for (int m = 0; m < QR; ++m) {
          const float4 q = *(const float4*)&q_lds[m * kHeadDim + 4 * c4];
          lg[m] = fmaf(x.x, q.x, lg[m]);
          lg[m] = fmaf(x.y, q.y, lg[m]);
          lg[m] = fmaf(x.z, q.z, lg[m]);
          lg[m] = fmaf(x.w, q.w, lg[m]);
        }
      }
    }
  }
  // the quad's four parts (a token's quad is all in or all past the slice)
  ds = f32_quad_sum(ds);
  if constexpr (!CAPT) {
#pragma unroll
    for (int m = 0; m < QR; ++m) lg[m] = f32_quad_sum(lg[m]);
  }
  if (i >= N || qp != 0) return;
  const float nrm = norms[srow + s0 + i];
  const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
  const float self = nrm > 0.f ? 1.f : 0.f;
  rowmean[srow + s0 + i] = (ds * inv - self) / (float)(N - 1);
  const int alpha = g.alpha;
  float best = 0.f;
  if constexpr (CAPT) {
    const float* a = imp_acc + (size_t)slice * g.G * g.capacity + s0 + i;
    best = a[0];
    for (int gq = 1; gq < g.G; ++gq) best = fmaxf(best, a[(size_t)gq * g.capacity]);
  } else {
    // weights of the token for each query row, summed over each GQA
    // member's alpha rows (consecutive), maximum over the members
    const float scale = 1.f / sqrtf((float)kHeadDim);
    float win = 0.f;
    int in_win = 0;
#pragma unroll
    for (int m = 0; m < QR; ++m) {
      const int pos = N - alpha + in_win;  // query row m's token
      const float w = (m < g.qrows && i <= pos) ? expf(lg[m] * scale - st_lds[m][0]) * st_lds[m][1] : 0.f;
      win += w;
      if (++in_win == alpha) {
        best = fmaxf(best, win);
        win = 0.f;
        in_win = 0;
      }
    }
  }
  importance[srow + s0 + i] = best / (float)alpha;
}

template <bool GATHER, bool CAPT, int QR>
static int launch_qr(const Geom& g, const LayerPtrs& k, const float* q, const int32_t* seq_start, const int32_t* order,
                     float* norms, float* parts, const float* imp_acc, float* importance, float* rowmean,
                     int32_t* counts, int slices, hipStream_t s) {
  RKV_LAUNCH((f32_stats_kernel<GATHER, CAPT, QR>), dim3(f32_chunks(g.n_slots), slices), dim3(kF32Threads), 0, s, g,
             k, q, seq_start, order, norms, parts, counts);
  RKV_LAUNCH((f32_pair_kernel<GATHER>), dim3(f32_tiles(g.n_slots), slices), dim3(kF32Threads), 0, s, g, k,
             seq_start, order, (const float*)norms, counts);
  RKV_LAUNCH((f32_final_kernel<GATHER, CAPT, QR>), dim3((g.n_slots + kF32FinalTok - 1) / kF32FinalTok, slices),
             dim3(kF32Threads), 0, s, g, k, q, seq_start, order, (const float*)norms, (const float*)parts, imp_acc,
             importance, rowmean);
  return 0;
}

template <bool GATHER, bool CAPT>
static int launch_f32_t(const Geom& g, const LayerPtrs& k, const float* q, const int32_t* seq_start,
                        const int32_t* order, float* norms, float* parts, float* importance, float* rowmean,
                        int32_t* counts, hipStream_t s, const float* imp_acc) {
  const int slices = g.L * g.batch * g.H;
  if constexpr (CAPT)
    return launch_qr<GATHER, true, 8>(g, k, q, seq_start, order, norms, parts, imp_acc, importance, rowmean, counts,
                                      slices, s);
  if (g.qrows <= 8)
    return launch_qr<GATHER, false, 8>(g, k, q, seq_start, order, norms, parts, imp_acc, importance, rowmean, counts,
                                       slices, s);
  if (g.qrows <= 16)
    return launch_qr<GATHER, false, 16>(g, k, q, seq_start, order, norms, parts, imp_acc, importance, rowmean, counts,
                                        slices, s);
  if (g.qrows <= 32)
    return launch_qr<GATHER, false, 32>(g, k, q, seq_start, order, norms, parts, imp_acc, importance, rowmean, counts,
                                        slices, s);
  return launch_qr<GATHER, false, 64>(g, k, q, seq_start, order, norms, parts, imp_acc, importance, rowmean, counts,
                                      slices, s);
}

int launch_score_f32(const Geom& g, const LayerPtrs& k, const void* obs_q, const int32_t* seq_start,
                     const int32_t* order, float* norms, float* parts, float* importance, float* rowmean,
                     int32_t* counts, void* stream, const float* imp_acc) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0 || g.n_slots <= g.budget) return 0;
  if ((order && imp_acc) || !norms || !parts || g.qrows > RKV_MAX_QROWS) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  const float* q = (const float*)obs_q;
  if (order) return launch_f32_t<true, false>(g, k, q, seq_start, order, norms, parts, importance, rowmean, counts, s,
                                              imp_acc);
  if (imp_acc) return launch_f32_t<false, true>(g, k, q, seq_start, order, norms, parts, importance, rowmean, counts,
                                                s, imp_acc);
  return launch_f32_t<false, false>(g, k, q, seq_start, order, norms, parts, importance, rowmean, counts, s, imp_acc);
}

}  // namespace rkv
