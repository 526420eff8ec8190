// Device-side building blocks of the gfx950 kernels: element types, key
// fragments in the MFMA operand layout, wave/block reductions and the
// XCD-aware work-group remap.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

#include "rkv_internal.hpp"

namespace rkv {

// Launches kernel(args...) and returns the launch's own hipError_t (0 =
// success). hipLaunchKernel reports the status of this launch; reading
// hipGetLastError after a triple-chevron launch would also return an error
// left behind by any earlier, unrelated HIP call of the thread.
template <typename... P, typename... A>
inline int launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> t(static_cast<P>(std::forward<A>(a))...);
  return std::apply(
      [&](auto&... x) {
        void* ptrs[] = {(void*)&x...};
        return (int)hipLaunchKernel((const void*)kernel, grid, block, ptrs, lds, stream);
      },
      t);
}
#define RKV_LAUNCH(...)                          \
  do {                                           \
    const int e_ = launch_kernel(__VA_ARGS__);   \
    if (e_ != 0) return e_;                      \
  } while (0)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Storage types: bf16 values travel as raw 16-bit patterns.
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
};
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
};

// One lane's half of a key row in the 32x32 MFMA operand layout: lane l holds
// dims [64*(l/32), 64*(l/32)+64) of key/query row (l % 32). Within a k-step
// the hardware pairs operand lanes by l/32, so A and B fragments built the
// same way contract the same dimension order; the order of the 128 dims is a
// permutation of the dot product's terms.
template <typename T>
struct Frag {
  static constexpr int kU4 = 64 * Elem<T>::kBytes / 16;  // 8 for bf16, 16 for f32
  uint4 v[kU4];
};

__device__ inline float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// The 64 values of a fragment as fp32 (exact widening).
template <typename T>
__device__ inline float frag_val(const Frag<T>& f, int e);
template <>
__device__ inline float frag_val<bf16_t>(const Frag<bf16_t>& f, int e) {
  const uint32_t w = ((const uint32_t*)&f.v[e >> 3])[(e & 7) >> 1];
  return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}
template <>
__device__ inline float frag_val<float>(const Frag<float>& f, int e) {
  return __uint_as_float(((const uint32_t*)&f.v[e >> 2])[e & 3]);
}

// Negates every value of a fragment (flips the sign bits).
template <typename T>
__device__ inline void frag_negate(Frag<T>& f) {
  const uint32_t m = sizeof(T) == 2 ? 0x80008000u : 0x80000000u;
#pragma unroll
  for (int i = 0; i < Frag<T>::kU4; ++i) f.v[i] = make_uint4(f.v[i].x ^ m, f.v[i].y ^ m, f.v[i].z ^ m, f.v[i].w ^ m);
}

template <typename T>
__device__ inline void frag_zero(Frag<T>& f) {
#pragma unroll
  for (int i = 0; i < Frag<T>::kU4; ++i) f.v[i] = make_uint4(0, 0, 0, 0);
}

// Loads one lane's half row: `half_row` points at the lane's 64 values.
template <typename T>
__device__ inline void frag_load(Frag<T>& f, const void* half_row) {
  const uint4* p = (const uint4*)half_row;
#pragma unroll
  for (int i = 0; i < Frag<T>::kU4; ++i) f.v[i] = p[i];
}

// acc += A-row fragment x B-column fragment over all 128 dims.
__device__ inline void mma_frag(f32x16& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v[s]),
                                                  __builtin_bit_cast(bf16x8_t, b.v[s]), acc, 0, 0, 0);
}
__device__ inline void mma_frag(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const float* x = (const float*)&a.v[s];
    const float* y = (const float*)&b.v[s];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x[e], y[e], acc, 0, 0, 0);
  }
}

// s_waitcnt immediate for vmcnt(v), other counters unconstrained (gfx9 encoding).
__device__ constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

// Raw buffer descriptors: base address, byte extent and the gfx9 descriptor
// word 3 for 32-bit raw access (stride 0, no swizzle). Accesses past the
// extent are range-checked per dword by the hardware: loads return 0 (also
// into LDS) without touching memory, so ragged tails need no clamping.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kRawBufferWord3 = 0x00020000u;

__device__ inline u32x4_t make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4_t d;
  d.x = (uint32_t)a;
  d.y = (uint32_t)(a >> 32) & 0xFFFFu;
  d.z = bytes;
  d.w = kRawBufferWord3;
  return d;
}

// The same extent as a resource the compiler's own buffer intrinsics take
// (their loads and stores are tracked by the compiler's memory counters).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRawBufferWord3);
}

// LDS byte address of a shared-memory pointer (uniform across the wave).
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct buffer-to-LDS loads: lane l writes lds + 16*l (or + 4*l) with the
// bytes at voff + soff of the buffer. Issued from inline assembly on purpose:
// the compiler cannot tell which LDS bytes such a load writes, so for the
// builtin it makes every later LDS read wait for all of them (vmcnt(0)),
// which would serialise a multi-stage ring. The caller orders them with
// explicit vmcnt waits and barriers instead; the loads count in vmcnt like
// any vector memory load. M0 holds the LDS base; one wait state separates
// its write from the load that reads it.
__device__ inline void dma_to_lds16(u32x4_t desc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(desc), "s"(soff)
      : "memory", "m0");
}
__device__ inline void dma_to_lds4(u32x4_t desc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(desc), "s"(soff)
      : "memory", "m0");
}

// Row of the 32x32 MFMA result held in accumulator register r of a lane in
// half `hh` (= lane / 32); the column is lane % 32.
__device__ inline int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// Work-groups are dispatched round-robin over the 8 XCDs; remap the hardware
// id so that consecutive logical work items share an XCD (and its L2).
__device__ inline int xcd_remap(int bid, int nblocks) {
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int per = nblocks / kXcds, rem = nblocks % kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

__device__ inline void slice_coords(const Geom& g, int slice, int& l, int& b, int& h) {
  h = slice % g.H;
  b = (slice / g.H) % g.batch;
  l = slice / (g.H * g.batch);
}

// First valid slot and valid-token count of sequence b, with seq_start
// clamped into [0, n_slots].
__device__ inline void seq_range(const Geom& g, const int32_t* seq_start, int b, int& s0, int& N) {
  int s = seq_start[b];
  s = s < 0 ? 0 : (s > g.n_slots ? g.n_slots : s);
  s0 = s;
  N = g.n_slots - s;
}

template <typename T>
__device__ inline const char* row_ptr(const void* layer, const Geom& g, int b, int h, int slot) {
  return (const char*)layer + (((size_t)b * g.H + h) * g.capacity + slot) * (size_t)(kHeadDim * Elem<T>::kBytes);
}

// The value of lane ^ 32 (or lane ^ 16) of a wave, from gfx950's lane-swap
// instructions: VALU operations, where a general shuffle is an LDS round trip
// (ds_bpermute). permlane32_swap(a, b) exchanges lanes 32..63 of a with lanes
// 0..31 of b; with a = b = v its two results hold v's low half twice and its
// high half twice, and the partner of a lane is the one its own half does not
// hold. permlane16_swap does the same between the odd and even 16-lane rows.
// The exec mask must be full (every caller is wave-uniform there).
__device__ inline uint32_t lane_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ inline uint32_t lane_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}
__device__ inline float lane_xor32(float v) { return __uint_as_float(lane_xor32(__float_as_uint(v))); }
__device__ inline float lane_xor16(float v) { return __uint_as_float(lane_xor16(__float_as_uint(v))); }
// v + v[lane ^ 32] and max(v, v[lane ^ 32]): the swap's two results are the
// lane's own value and its partner's, in some order, so no select is needed
// (addition and max are commutative: the same bits as with the partner).
__device__ inline float xor32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline uint32_t xor32_add(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] + r[1];
}
__device__ inline float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor16_add(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// v + v[lane ^ 8]: within a 16-lane row, rotating by 8 is the xor
__device__ inline float xor8_add(float v) {
  return v + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x128 /* row_ror:8 */, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave in DPP steps (no LDS
// round trips): within each 16-lane row, shifts by 1, 2 and 3, then by 4 and
// 8 on the banks that have a source; then the last lane of each even row is
// added into the next row (row_bcast:15), and lane 31 into rows 2 and 3
// (row_bcast:31). Lanes a step does not write add 0. The exec mask must be
// full.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ inline int dpp_add_src(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, false);
}
__device__ inline int wave_prefix_sum(int x) {
  int s = x + dpp_add_src<0x111, 0xF, 0xF>(x);  // row_shr:1
  s += dpp_add_src<0x112, 0xF, 0xF>(x);         // row_shr:2
  s += dpp_add_src<0x113, 0xF, 0xF>(x);         // row_shr:3
  s += dpp_add_src<0x114, 0xF, 0xE>(s);         // row_shr:4, lanes 4..15 of each row
  s += dpp_add_src<0x118, 0xF, 0xC>(s);         // row_shr:8, lanes 8..15 of each row
  s += dpp_add_src<0x142, 0xA, 0xF>(s);         // row_bcast:15 into rows 1 and 3
  s += dpp_add_src<0x143, 0xC, 0xF>(s);         // row_bcast:31 into rows 2 and 3
  return s;
}

// Sum over the 64 lanes, every lane receiving it: DPP within each 16-lane
// row (lanes 1 and 2 apart in a quad, the mirrored quad of each 8, the
// mirrored 8 of the row), then the half swaps across rows and halves. Each
// step adds two partial sums that its two partners hold alike, so every lane
// ends with the same bits. The exec mask must be full.
__device__ inline float wave_sum(float v) {
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1, 0, 3, 2]
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2, 3, 0, 1]
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x140, 0xF, 0xF, false));  // row_mirror
  v = xor16_add(v);
  return xor32_add(v);
}

// Exclusive prefix sum over the block in thread order; *total receives the
// block total. scratch holds 16 ints.
__device__ inline int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int x = wave_prefix_sum(v);  // inclusive, within the wave
  __syncthreads();
  if (lane == 63) scratch[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < w) before += scratch[i];
    tot += scratch[i];
  }
  *total = tot;
  return before + x - v;
}

}  // namespace rkv
