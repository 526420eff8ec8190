// Building blocks of the scoring kernels shared by the pair kernel
// (rkv_score.hip) and the gathered scoring kernel of the hole-filling layout
// (rkv_gram.hip): staged key rows in LDS, MFMA fragments read from them, the
// similar-pair sign-bit test, the sum of unit keys as MFMA rows, softmax
// statistics merges and vector-memory waits.
#pragma once

#include "rkv_device.hpp"

namespace rkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Key rows staged in LDS: row R at R * kRowBytes, its 16-byte slot p holding
// the row's bytes [16 (p ^ (R & 15)), +16) (XOR swizzle: the MFMA operand
// reads of 32 consecutive rows hit distinct banks).
template <typename T>
struct Row {
  static constexpr int kBytes = kHeadDim * Elem<T>::kBytes;  // 256 (bf16) or 512 (fp32)
  static constexpr int kSlots = kBytes / 16;
};

// Waits until at most n of this wave's vector memory operations are
// outstanding (n clamped to [0, 31], which only waits longer).
__device__ inline void wait_vm(int n) {
  switch (n < 0 ? 0 : (n < 31 ? n : 31)) {
#define RKV_VM_CASE(i) \
  case i:              \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(i)); break;
    RKV_VM_CASE(0) RKV_VM_CASE(1) RKV_VM_CASE(2) RKV_VM_CASE(3) RKV_VM_CASE(4) RKV_VM_CASE(5) RKV_VM_CASE(6)
    RKV_VM_CASE(7) RKV_VM_CASE(8) RKV_VM_CASE(9) RKV_VM_CASE(10) RKV_VM_CASE(11) RKV_VM_CASE(12)
    RKV_VM_CASE(13) RKV_VM_CASE(14) RKV_VM_CASE(15) RKV_VM_CASE(16) RKV_VM_CASE(17) RKV_VM_CASE(18)
    RKV_VM_CASE(19) RKV_VM_CASE(20) RKV_VM_CASE(21) RKV_VM_CASE(22) RKV_VM_CASE(23) RKV_VM_CASE(24)
    RKV_VM_CASE(25) RKV_VM_CASE(26) RKV_VM_CASE(27) RKV_VM_CASE(28) RKV_VM_CASE(29) RKV_VM_CASE(30)
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(31)); break;
#undef RKV_VM_CASE
  }
}

// MFMA operand fragment (32x32 layout) of staged row R, the lane's half hh.
template <typename T>
__device__ inline void frag_from_stage(Frag<T>& f, const char* st_rows, int R, int hh) {
  const char* row = st_rows + R * Row<T>::kBytes;
  const int sw = R & 15;
#pragma unroll
  for (int s = 0; s < Frag<T>::kU4; ++s) f.v[s] = *(const uint4*)(row + (((hh * (Row<T>::kSlots / 2) + s) ^ sw) * 16));
}

// Merges the softmax statistics (m2, s2) into (m1, s1).
__device__ inline void merge_ms(float& m1, float& s1, float m2, float s2) {
  const float m = fmaxf(m1, m2);
  if (m == -INFINITY) return;
  s1 = (m1 > -INFINITY ? s1 * __expf(m1 - m) : 0.f) + (m2 > -INFINITY ? s2 * __expf(m2 - m) : 0.f);
  m1 = m;
}

// Similar pairs of one 32x32 tile: d = tau|k_i| |k_j| - G_ij is negative iff
// S_ij > tau; each sign bit is shifted into a per-lane mask (one alignbit per
// element, no compare / carry chain), whose bits are counted once per block.
__device__ inline uint32_t sign_bits(const f32x16& acc, float tn, const float* nj, uint32_t mask) {
#pragma unroll
  for (int r = 0; r < 16; ++r) mask = __builtin_amdgcn_alignbit(mask, __float_as_uint(fmaf(tn, nj[r], -acc[r])), 31);
  return mask;
}
// The count on the diagonal tile: only pairs whose row (newer token, index
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
  static constexpr int ROWS = 3;
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
  static constexpr int ROWS = 1;
  __device__ static void write(char* tile, int d, float s) {
    const int byte = d * 4;
    *(float*)(tile + ((byte >> 4) << 4) + (byte & 15)) = s;  // row 0: no swizzle
  }
  __device__ static float dot(const f32x16& acc) { return acc[0]; }
};

}  // namespace rkv
