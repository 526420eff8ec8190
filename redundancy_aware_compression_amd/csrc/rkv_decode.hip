// Decode attention with importance capture. R-KV scores each cached token by
// the attention that the newest alpha queries pay it (R-KV notes page,
// summary table row "importance computation"), and the notes name fusing
// attention, importance scoring and eviction into one kernel as the way to
// cut the cost of compression (Q&A part 2, cause 4). The decode step already
// computes those attention rows: this kernel computes the newest token's
// attention output and, during the alpha steps before an eviction, adds each
// query head's normalised weights into a per-slot accumulator. The eviction
// step then reads its importance from the accumulator instead of recomputing
// the observation queries' attention.
#include "rkv_device.hpp"

namespace rkv {

// Work-groups of 512 threads, or 256 where the weights leave room in LDS for
// three of them per compute unit (short slices) and there are slices enough
// for several per unit: more waves per unit then.
constexpr size_t kDecSmallLds = 40 * 1024;

// A lane holds one 16-byte chunk of a row: LPR lanes cover a row, RPI rows
// are covered by one load instruction of the wave (fully coalesced). dot()
// is the lane's part of q.k: bf16 pairs go to the packed dot instruction
// unwidened (exact products, fp32 sums) and the scale comes after the row
// sum; fp32 queries are pre-scaled.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <typename T>
struct DecLanes;
template <>
struct DecLanes<bf16_t> {
  static constexpr int LPR = 16, EPL = 8;
  static constexpr bool PRESCALED = false;
  using QV = uint4;
  __device__ static QV load_q(const char* p, float) { return *(const uint4*)p; }
  __device__ static float d2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
  }
  __device__ static float dot(const uint4& k, const QV& q) {
    return d2(k.w, q.w, d2(k.z, q.z, d2(k.y, q.y, d2(k.x, q.x, 0.f))));
  }
  __device__ static void widen(const uint4& x, float* f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct DecLanes<float> {
  static constexpr int LPR = 32, EPL = 4;
  static constexpr bool PRESCALED = true;
  using QV = float4;
  __device__ static QV load_q(const char* p, float scale) {
    float4 q = *(const float4*)p;
    return make_float4(q.x * scale, q.y * scale, q.z * scale, q.w * scale);
  }
  __device__ static float dot(const uint4& k, const QV& q) {
    float s = __uint_as_float(k.x) * q.x;
    s = fmaf(__uint_as_float(k.y), q.y, s);
    s = fmaf(__uint_as_float(k.z), q.z, s);
    return fmaf(__uint_as_float(k.w), q.w, s);
  }
  __device__ static void widen(const uint4& x, float* f) {
    f[0] = __uint_as_float(x.x);
    f[1] = __uint_as_float(x.y);
    f[2] = __uint_as_float(x.z);
    f[3] = __uint_as_float(x.w);
  }
};

// Sum over the LPR lanes of a row: quad swaps, half-row and row mirrors
// (every lane of the 16 receives the total), then lanes 16 apart for fp32.
template <int LPR>
__device__ inline float row_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  if constexpr (LPR == 32) v = xor16_add(v);
  return v;
}

// The element of a G-register array selected by a runtime index, as a chain
// of selects. Each element passes through an empty asm so that the chain
// cannot be turned back into an indexed access, which would put the array in
// scratch memory.
template <int G>
__device__ inline float pick(const float (&a)[G], int i) {
  float r = a[0];
#pragma unroll
  for (int k = 1; k < G; ++k) {
    float ak = a[k];
    asm volatile("" : "+v"(ak));
    r = i == k ? ak : r;
  }
  return r;
}

// One work-group per slice (layer, sequence, KV head) with N valid slots
// [s0, n_slots): for each of its G query heads, w = softmax over the N keys
// of q.k / sqrt(D) and out = sum_j w_j v_j (fp32). With acc, the weights are
// added to acc[slice][g][s0 + j]. LDS (dynamic): the logits, then the
// weights, as [N][G]; afterwards the waves' partial outputs [8][G][128].
template <typename T, int G, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(Geom g, LayerPtrs k, LayerPtrs v,
                                                             const void* __restrict__ q,
                                                             const int32_t* __restrict__ seq_start,
                                                             float* __restrict__ out, float* __restrict__ acc) {
  using DL = DecLanes<T>;
  constexpr int LPR = DL::LPR, EPL = DL::EPL, RPI = 64 / LPR;
  constexpr int RB = kHeadDim * (int)sizeof(T);
  constexpr int NW = NT / 64;
  constexpr int U = 4;  // row loads per lane per round (two rounds in flight)
  constexpr int STEP = NW * RPI * U;  // rows per round of the work-group
  extern __shared__ __align__(16) float lw[];
  __shared__ float red_m[NW][G], red_s[NW][G];

  const int slice = blockIdx.x;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  seq_range(g, seq_start, b, s0, N);
  const int tid = threadIdx.x, lane = tid & 63, c = lane % LPR, rr = lane / LPR;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the row loops branch on scalars
  float* o_out = out + (size_t)slice * G * kHeadDim;
  if (N == 0) {
    for (int e = tid; e < G * kHeadDim; e += NT) o_out[e] = 0.f;
    return;
  }
  const char* kb = row_ptr<T>(k.p[l], g, b, h, s0);
  const char* vb = row_ptr<T>(v.p[l], g, b, h, s0);

  // the lane's chunk of each query row; logits are in log2 units
  const float qs = 1.4426950408889634f / sqrtf((float)kHeadDim);
  typename DL::QV qv[G];
  {
    const char* qb = (const char*)q + (size_t)slice * G * RB;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) qv[gi] = DL::load_q(qb + gi * RB + c * 16, qs);
  }

  // Rounds of U loads per lane, software-pipelined: the next round is issued
  // before the current one is used, and the K pass's last prefetch is the V
  // pass's first round, so those loads fly across the softmax below. Each
  // round is a buffer load through a descriptor rebased to its first row (a
  // few scalar operations) with the extent of the rows left, so rows past the
  // slice read as zeros without touching memory, and the per-lane offsets are
  // loop-invariant: no vector temporaries that could share registers with a
  // load still in flight.
  uint32_t voff[U];
#pragma unroll
  for (int u = 0; u < U; ++u) voff[u] = (uint32_t)(u * RPI + rr) * RB + (uint32_t)c * 16u;
  auto load_round = [&](uint4(&x)[U], const char* base, int j0) {
    const int left = N - j0;  // uniform
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (size_t)j0 * RB, left > 0 ? (uint32_t)left * RB : 0u);
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[u], 0, 0));
  };
  const int jstart = wave * RPI * U;
  uint4 xa[U], xb[U];
  load_round(xa, kb, jstart);

  // ---- logits: lane c < G of each row stores query c's logit and keeps its max.
  // The two buffers alternate (no copy from one to the other: a copy would
  // wait for the prefetch and leave one round in flight).
  float mrun = -INFINITY;
  auto k_round = [&](const uint4(&cur)[U], uint4(&nxt)[U], int j0) {
    const int jn = j0 + STEP;
    load_round(nxt, jn < N ? kb : vb, jn < N ? jn : jstart);
    __builtin_amdgcn_sched_barrier(0);  // the next round's loads go out before this round's work
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float part[G];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) part[gi] = row_sum<LPR>(DL::dot(cur[u], qv[gi]));
      const int row = j0 + u * RPI + rr;
      if (c < G && row < N) {
        const float lg = DL::PRESCALED ? pick<G>(part, c) : pick<G>(part, c) * qs;
        lw[row * G + c] = lg;
        mrun = fmaxf(mrun, lg);
      }
    }
  };
  bool v_in_b = false;  // the buffer that holds the V pass's first round
  for (int j0 = jstart; j0 < N; j0 += 2 * STEP) {
    k_round(xa, xb, j0);
    if (j0 + STEP >= N) {
      v_in_b = true;
      break;
    }
    k_round(xb, xa, j0 + STEP);
  }
  if constexpr (LPR == 16) mrun = xor16_max(mrun);  // the rows of the wave (lanes LPR apart)
  mrun = xor32_max(mrun);
  if (rr == 0 && c < G) red_m[wave][c] = mrun;
  __syncthreads();
  float m[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = red_m[0][gi];
#pragma unroll
    for (int w = 1; w < NW; ++w) m[gi] = fmaxf(m[gi], red_m[w][gi]);
  }

  // ---- weights (unnormalised) and their sums, by rows: the G weights of a
  // row are contiguous, and each thread reads RW rows before it computes, so
  // the LDS round trips overlap
  float ssum[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) ssum[gi] = 0.f;
  constexpr int RW = 4;
  for (int j0 = tid; j0 < N; j0 += RW * NT) {
    float lv[RW][G];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int j = min(j0 + r * NT, N - 1);  // in range; rows past N are not used
#pragma unroll
      for (int gi = 0; gi < G; ++gi) lv[r][gi] = lw[j * G + gi];
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int j = j0 + r * NT;
      if (j < N) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const float p = exp2f(lv[r][gi] - m[gi]);
          lw[j * G + gi] = p;
          ssum[gi] += p;
        }
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const float s = wave_sum(ssum[gi]);
    if (lane == 0) red_s[wave][gi] = s;
  }
  __syncthreads();  // the weights are in LDS and the sums in red_s
  float inv[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red_s[w][gi];
    inv[gi] = 1.f / s;
  }

  // ---- output: o[g] = sum_j p_j v_j over the lane's rows and dims (xa or xb
  // holds the first round of V)
  float o[G][EPL];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[gi][e] = 0.f;
  auto v_round = [&](const uint4(&cur)[U], uint4(&nxt)[U], int j0) {
    load_round(nxt, vb, j0 + STEP);  // rows past the slice read as zeros
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = j0 + u * RPI + rr;
      const bool ok = row < N;
      const int rc = ok ? row : N - 1;  // in-bounds LDS index for rows past the slice (zero rows, weight 0)
      float vf[EPL];
      DL::widen(cur[u], vf);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float p = ok ? lw[rc * G + gi] : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[gi][e] = fmaf(p, vf[e], o[gi][e]);
      }
    }
  };
  auto v_pass = [&](uint4(&x0)[U], uint4(&x1)[U]) {
    for (int j0 = jstart; j0 < N; j0 += 2 * STEP) {
      v_round(x0, x1, j0);
      if (j0 + STEP >= N) break;
      v_round(x1, x0, j0 + STEP);
    }
  };
  // one V loop, starting from xa. Its first round had the whole softmax to
  // land: wait for it here, so that no load is pending into the loop and the
  // loop header needs no wait of its own
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (v_in_b) {
#pragma unroll
    for (int u = 0; u < U; ++u) xa[u] = xb[u];
  }
  v_pass(xa, xb);

  // ---- capture: acc[g][j] += w_gj. Every query's accumulator loads for a
  // batch of rows go out together (one memory round trip per batch, not per
  // query); CU rows per thread keep the batch near 16 values.
  if (acc) {
    constexpr int CU = 16 / G > 0 ? 16 / G : 1;
    float* ab = acc + (size_t)slice * G * g.capacity + s0;  // [G][capacity] from the slice's first valid slot
    for (int j0 = tid; j0 < N; j0 += CU * NT) {
      float a[G][CU];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int j = min(j0 + u * NT, N - 1);  // in range; rows past N are not used
#pragma unroll
        for (int gi = 0; gi < G; ++gi) a[gi][u] = ab[(size_t)gi * g.capacity + j];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int j = j0 + u * NT;
        if (j < N) {
#pragma unroll
          for (int gi = 0; gi < G; ++gi) ab[(size_t)gi * g.capacity + j] = fmaf(lw[j * G + gi], inv[gi], a[gi][u]);
        }
      }
    }
  }

  // ---- combine the rows of the wave, then the waves
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if constexpr (LPR == 16) o[gi][e] = xor16_add(o[gi][e]);
      o[gi][e] = xor32_add(o[gi][e]);
    }
  __syncthreads();  // every wave is done with the weights
  if (rr == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int e = 0; e < EPL; ++e) lw[(wave * G + gi) * kHeadDim + c * EPL + e] = o[gi][e];
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += NT) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += lw[w * G * kHeadDim + e];
    o_out[e] = s * pick<G>(inv, e / kHeadDim);
  }
}

template <typename T, int G, int NT>
static int launch_decode_nt(const Geom& g, const LayerPtrs& k, const LayerPtrs& v, const void* q,
                            const int32_t* seq_start, float* out, float* acc, hipStream_t s, size_t lds) {
  if (lds > 65536) {
    const int err = (int)hipFuncSetAttribute((const void*)decode_kernel<T, G, NT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err) return err;
  }
  RKV_LAUNCH((decode_kernel<T, G, NT>), dim3(g.L * g.batch * g.H), dim3(NT), lds, s, g, k, v, q,
                     seq_start, out, acc);
  return 0;
}

template <typename T, int G>
static int launch_decode_g(const Geom& g, const LayerPtrs& k, const LayerPtrs& v, const void* q,
                           const int32_t* seq_start, float* out, float* acc, hipStream_t s) {
  const size_t lds = decode_lds_bytes(G, g.n_slots);
  const bool small = lds <= kDecSmallLds && g.L * g.batch * g.H >= 4 * kCUs;
  return small ? launch_decode_nt<T, G, 256>(g, k, v, q, seq_start, out, acc, s, lds)
               : launch_decode_nt<T, G, 512>(g, k, v, q, seq_start, out, acc, s, lds);
}

template <typename T>
static int launch_decode_t(const Geom& g, const LayerPtrs& k, const LayerPtrs& v, const void* q,
                           const int32_t* seq_start, float* out, float* acc, hipStream_t s) {
  switch (g.G) {
    case 1: return launch_decode_g<T, 1>(g, k, v, q, seq_start, out, acc, s);
    case 2: return launch_decode_g<T, 2>(g, k, v, q, seq_start, out, acc, s);
    case 3: return launch_decode_g<T, 3>(g, k, v, q, seq_start, out, acc, s);
    case 4: return launch_decode_g<T, 4>(g, k, v, q, seq_start, out, acc, s);
    case 5: return launch_decode_g<T, 5>(g, k, v, q, seq_start, out, acc, s);
    case 6: return launch_decode_g<T, 6>(g, k, v, q, seq_start, out, acc, s);
    case 7: return launch_decode_g<T, 7>(g, k, v, q, seq_start, out, acc, s);
    case 8: return launch_decode_g<T, 8>(g, k, v, q, seq_start, out, acc, s);
    default: return (int)hipErrorInvalidValue;
  }
}

int launch_decode(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const void* q,
                  const int32_t* seq_start, float* out, float* acc, void* stream) {
  if (g.L * g.batch * g.H == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  return dtype == RKV_BF16 ? launch_decode_t<bf16_t>(g, k, v, q, seq_start, out, acc, s)
                           : launch_decode_t<float>(g, k, v, q, seq_start, out, acc, s);
}

}  // namespace rkv
