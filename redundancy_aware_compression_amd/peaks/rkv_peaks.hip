// Peak microbenchmarks for the roofline figures of the eviction kernels: the
// bf16 MFMA issue rate of the chip and its HBM read and copy bandwidth, as
// measured by plain kernels (the rooflines quote MI355X's published peaks;
// these show how close a plain kernel gets to them).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv_peaks.h"

namespace {

constexpr int kThreads = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Four independent 32x32x16 bf16 MFMA chains per wave, `iters` rounds: one
// MFMA issue every time the matrix pipe of the SIMD is free. One float per
// lane is written so the chains are not removed.
//
// The matrix units draw more power on operands whose bits change (signs,
// exponents, mantissas) than on repetitive ones, and under that load the
// chip lowers its clock. LOW: few distinct small values from the lane id,
// which keeps the clock up and approaches the published rate. RANDOM: every
// lane's 16 operands are bf16 values of random sign, exponent in [2^-2, 2^2)
// and random mantissa (about what keys drawn from N(0, 1) look like), from a
// xorshift generator seeded by lane and work-group: the rate a kernel on
// real keys can reach at best.
template <bool RANDOM>
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(int iters, float* __restrict__ out) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
  uint32_t h = ((uint32_t)tid + 1u) * 2654435761u ^ ((uint32_t)blockIdx.x + 1u) * 40503u;
  auto next = [&]() {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    return h;
  };
  auto rand_bf16 = [&]() {
    const uint32_t r = next();
    return __builtin_bit_cast(__bf16, (uint16_t)((r & 0x8000u) | ((125u + ((r >> 20) & 3u)) << 7) | (r & 0x7Fu)));
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (RANDOM) {
      a[i] = rand_bf16();
      b[i] = rand_bf16();
    } else {
      a[i] = (__bf16)(0.001f * (float)((tid + i) & 7));
      b[i] = (__bf16)(0.002f * (float)((tid ^ i) & 7));
    }
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * kThreads + tid] = s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Tiles of kUnroll * kThreads 16-byte words (32 KiB) go to the work-groups
// in turn; a work-group reads a tile with kUnroll coalesced non-temporal
// loads per thread in flight, and folds it with XOR into one word per block.
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                            uint32_t* __restrict__ out) {
  __shared__ uint32_t red[kThreads / 64];
  constexpr size_t TILE = (size_t)kUnroll * kThreads;
  const size_t ntiles = n16 / TILE;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const u32x4* p = src + t * TILE + threadIdx.x;
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(p + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  for (size_t i = ntiles * TILE + (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kThreads)
    acc ^= __builtin_nontemporal_load(&src[i]);
  uint32_t a = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a ^= __shfl_xor(a, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// dst = src over n16 16-byte words, by the same 32 KiB tiles: kUnroll
// non-temporal loads per thread, then their stores.
__global__ __launch_bounds__(kThreads) void hbm_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            size_t n16) {
  constexpr size_t TILE = (size_t)kUnroll * kThreads;
  const size_t ntiles = n16 / TILE;
  for (size_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const size_t base = t * TILE + threadIdx.x;
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(&src[base + u * kThreads]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(x[u], &dst[base + u * kThreads]);
  }
  for (size_t i = ntiles * TILE + (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kThreads)
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

}  // namespace

extern "C" {

int rkv_peak_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  void* args[] = {&iters, &out};
  return (int)hipLaunchKernel((const void*)mfma_peak_kernel<false>, dim3(blocks), dim3(kThreads), args, 0,
                              (hipStream_t)stream);
}

int rkv_peak_mfma_bf16_random(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  void* args[] = {&iters, &out};
  return (int)hipLaunchKernel((const void*)mfma_peak_kernel<true>, dim3(blocks), dim3(kThreads), args, 0,
                              (hipStream_t)stream);
}

int rkv_peak_hbm_read(const void* src, size_t bytes, int32_t blocks, uint32_t* out, void* stream) {
  if (!src || !out || blocks < 1 || (bytes & 15u) || ((uintptr_t)src & 15u)) return (int)hipErrorInvalidValue;
  const u32x4* s4 = (const u32x4*)src;
  size_t n = bytes / 16;
  void* args[] = {&s4, &n, &out};
  return (int)hipLaunchKernel((const void*)hbm_read_kernel, dim3(blocks), dim3(kThreads), args, 0, (hipStream_t)stream);
}

int rkv_peak_hbm_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream) {
  if (!src || !dst || blocks < 1 || (bytes & 15u) || (((uintptr_t)src | (uintptr_t)dst) & 15u))
    return (int)hipErrorInvalidValue;
  const u32x4* s4 = (const u32x4*)src;
  u32x4* d4 = (u32x4*)dst;
  size_t n = bytes / 16;
  void* args[] = {&s4, &d4, &n};
  return (int)hipLaunchKernel((const void*)hbm_copy_kernel, dim3(blocks), dim3(kThreads), args, 0, (hipStream_t)stream);
}

int rkv_peak_threads_per_block(void) { return kThreads; }

}  // extern "C"
