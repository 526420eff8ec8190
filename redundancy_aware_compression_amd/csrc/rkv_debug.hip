// RKV_DEBUG device checks of the data preconditions the kernels rely on but
// cannot check without a host sync (see the Errors and Debug checks notes of
// include/rkv.h): seq_start within [0, n_slots], finite key, value and
// query elements in the slots a step reads, and (the hole-filling layout)
// each slice's order table a permutation of [0, budget). One work-group per
// slice ORs violation bits into flags[0] (vector atomics); every read stays
// inside the caller's buffers (seq_start clamped, order entries used only
// after their range check).
#include "rkv_device.hpp"

namespace rkv {

constexpr int kDbgThreads = 256;

__global__ void debug_clear_kernel(uint32_t* flags) {
  if (threadIdx.x == 0) flags[0] = 0u;
}

// Whether every element of the 16-byte word is finite (all-ones exponent:
// inf or NaN).
template <typename T>
__device__ inline bool word_finite(uint4 w) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (sizeof(T) == 2)
      ok = ok && (x[i] & 0x7F80u) != 0x7F80u && (x[i] & 0x7F800000u) != 0x7F800000u;
    else
      ok = ok && (x[i] & 0x7F800000u) != 0x7F800000u;
  }
  return ok;
}

template <typename T>
__global__ __launch_bounds__(kDbgThreads) void debug_check_kernel(Geom g, LayerPtrs k, LayerPtrs v, bool has_v,
                                                                  const void* __restrict__ obs_q,
                                                                  const int32_t* __restrict__ seq_start,
                                                                  const int32_t* __restrict__ order,
                                                                  uint32_t* __restrict__ flags) {
  extern __shared__ uint32_t seen[];  // order check: one bit per slot of [0, budget)
  constexpr int RB = kHeadDim * Elem<T>::kBytes, W = RB / 16;
  const int slice = blockIdx.x, tid = threadIdx.x;
  int l, b, h, s0, N;
  slice_coords(g, slice, l, b, h);
  uint32_t bad = 0u;
  if (l == 0 && h == 0 && tid == 0) {
    const int s = seq_start[b];
    if (s < 0 || s > g.n_slots) bad |= kDbgSeqStart;
  }
  seq_range(g, seq_start, b, s0, N);
  const int32_t* ord = order ? order + (size_t)slice * g.budget : nullptr;
  bool order_ok = true;
  if (ord) {
    for (int i = tid; i < (g.budget + 31) / 32; i += kDbgThreads) seen[i] = 0u;
    __syncthreads();
    for (int i = tid; i < g.budget; i += kDbgThreads) {
      const int o = ord[i];
      if (o < 0 || o >= g.budget) {
        order_ok = false;
      } else if (atomicOr(&seen[o >> 5], 1u << (o & 31)) & (1u << (o & 31))) {
        order_ok = false;  // a slot named twice
      }
    }
    if (!order_ok) bad |= kDbgOrder;
  }
  // the valid slots' rows (through the order table when it holds, virtual
  // slot v < budget at physical slot order[v])
  bool kv_ok = true;
  for (int e = tid; e < N * W; e += kDbgThreads) {
    const int vs = s0 + e / W;
    int phys = vs;
    if (ord && vs < g.budget) {
      const int o = ord[vs];
      phys = (o >= 0 && o < g.budget) ? o : vs;
    }
    const size_t off = (size_t)phys * RB + (size_t)(e % W) * 16;
    const uint4 kw = *(const uint4*)(row_ptr<T>(k.p[l], g, b, h, 0) + off);
    kv_ok = kv_ok && word_finite<T>(kw);
    if (has_v) {
      const uint4 vw = *(const uint4*)(row_ptr<T>(v.p[l], g, b, h, 0) + off);
      kv_ok = kv_ok && word_finite<T>(vw);
    }
  }
  if (!kv_ok) bad |= kDbgKV;
  if (obs_q && N > g.budget) {
    const char* qb = (const char*)obs_q + (size_t)slice * g.qrows * RB;
    bool q_ok = true;
    for (int e = tid; e < g.qrows * W; e += kDbgThreads) q_ok = q_ok && word_finite<T>(*(const uint4*)(qb + (size_t)e * 16));
    if (!q_ok) bad |= kDbgQuery;
  }
  if (bad) atomicOr(flags, bad);
}

int launch_debug_check(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const void* obs_q,
                       const int32_t* seq_start, const int32_t* order, uint32_t* flags, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  RKV_LAUNCH(debug_clear_kernel, dim3(1), dim3(64), 0, s, flags);
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  const size_t lds = order ? (size_t)((g.budget + 31) / 32) * 4 : 0;
  const bool has_v = v.p[0] != nullptr;
  if (dtype == RKV_BF16)
    RKV_LAUNCH(debug_check_kernel<bf16_t>, dim3(slices), dim3(kDbgThreads), lds, s, g, k, v, has_v, obs_q,
               seq_start, order, flags);
  else
    RKV_LAUNCH(debug_check_kernel<float>, dim3(slices), dim3(kDbgThreads), lds, s, g, k, v, has_v, obs_q,
               seq_start, order, flags);
  return 0;
}

}  // namespace rkv
