// In-place, order-preserving compaction of one (slice, K|V) row block,
// shared by the compaction kernel and the fused eviction-step kernel.
//
// Safety of the in-place gather: keep is ascending with keep[j] >= j, so when
// destinations are processed in ascending chunks, a chunk's writes land below
// every source of every later chunk (which may therefore be loaded while the
// chunk stores), and its own sources are all read before any of its writes
// (its loads returned in every thread, then a barrier, then its stores).
// Rows with keep[j] == j are skipped. R-KV notes page
// (yoonschallenge.tistory.com/1236), Q&A part 2, cause 3: the selected KV is
// copied into the new cache; cause 4: re-allocation and re-arrangement after
// pruning are costs, avoided here by moving rows within the cache.
#pragma once

#include "rkv_device.hpp"

namespace rkv {

constexpr int kCompactThreads = 512;
constexpr int kCompactUnroll = 16;  // 16-byte loads in flight per thread per chunk (128 KB per work-group)

typedef unsigned int u32x4n __attribute__((ext_vector_type(4)));

// The copied rows are not read again by this kernel: both directions bypass
// the caches' retention (non-temporal), which leaves more of the HBM
// bandwidth to the streams.
__device__ inline u32x4n load_nt(const char* p) { return __builtin_nontemporal_load((const u32x4n*)p); }
__device__ inline void store_nt(char* p, u32x4n v) { __builtin_nontemporal_store(v, (u32x4n*)p); }

// A sequence's first valid slot after the compaction: the number of leading
// -1 entries of one of its keep rows (binary search; every row of the
// sequence has the same number).
__device__ inline int leading_unkept(const int32_t* krow, int B) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (krow[mid] < 0)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Row j of [0, budget) of the row block at `base` receives row krow[j]
// (krow[j] < 0, == j or >= n_slots: left as it is). Every thread of the
// work-group (kCompactThreads) takes part.
//
// Chunks of CH_ROWS destination rows go through two register buffers, and
// chunk c + 1's loads are issued before chunk c's stores, so the memory pipe
// does not drain at every chunk. That is safe because every source of chunk
// c + 1 lies at or past its first row, above every destination of chunk c;
// within a chunk, all of its loads (every thread's) complete before the
// barrier that precedes its stores. The keep entries of a chunk arrive one
// chunk ahead (one load per lane, handed to the lanes that need them by
// shuffles), so no data load waits for a keep entry issued just before it.
// Loads and stores are range-checked buffer accesses: lanes whose row does
// not move take an offset past the range, which the hardware drops (loads
// return zeros) without touching memory, so nothing branches around them.
template <typename T>
__device__ inline void compact_rows(char* base, const int32_t* __restrict__ krow, const Geom& g) {
  constexpr int RB = kHeadDim * Elem<T>::kBytes;
  constexpr int U4_ROW = RB / 16;                       // lanes per row
  constexpr int RPW = 64 / U4_ROW;                      // rows of a wave per load instruction
  constexpr int CHQ = kCompactThreads / U4_ROW;         // rows of the work-group per load instruction
  constexpr int CH_ROWS = CHQ * kCompactUnroll;         // rows per chunk
  constexpr uint32_t kOff = 0x80000000u;                // past any range: dropped
  constexpr int kNt = 2;                                // non-temporal cache policy
  const int B = g.budget, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (B + CH_ROWS - 1) / CH_ROWS;
  if (nch == 0) return;
  const __amdgpu_buffer_rsrc_t src_rs = make_rsrc(base, (uint32_t)g.n_slots * RB);
  const __amdgpu_buffer_rsrc_t dst_rs = make_rsrc(base, (uint32_t)B * RB);
  const int sub = lane / U4_ROW;                        // the lane's row within a load instruction of its wave
  const uint32_t part = (uint32_t)(lane % U4_ROW) * 16u;
  // the keep entry of row CHQ (L / RPW) + RPW wave + L % RPW of chunk c, for
  // lane L (rows past the budget read -1). A volatile load: the compiler
  // keeps it where it is issued, ahead of the stores, instead of sinking it
  // to its use, where waiting for it would also wait for every older access.
  const __amdgpu_buffer_rsrc_t keep_rs = make_rsrc(krow, (uint32_t)B * 4u);
  auto load_kr = [&](int c) {
    const int L = lane % (kCompactUnroll * RPW);
    const int r = c * CH_ROWS + CHQ * (L / RPW) + RPW * wave + L % RPW;
    return r < B ? __builtin_amdgcn_raw_buffer_load_b32(keep_rs, (uint32_t)r * 4u, 0, (int)(1u << 31)) : -1;
  };
  // Sixteen 16-byte loads per thread per chunk, held in named registers (an
  // array here is kept in scratch memory across the barrier by the compiler).
  static_assert(kCompactUnroll == 16, "the chunk bodies below are written out for 16 loads");
  struct Buf {
    u32x4n v0, v1, v2, v3, v4, v5, v6, v7, v8, v9, v10, v11, v12, v13, v14, v15;
    uint32_t d0, d1, d2, d3, d4, d5, d6, d7, d8, d9, d10, d11, d12, d13, d14, d15;  // destination offsets
  };
  // load q of chunk c: row c0 + CHQ q + RPW wave + sub, whose keep entry lane RPW q + sub holds
  auto load_chunk = [&](int c, int kr, Buf& x) {
    const int c0 = c * CH_ROWS;
    auto ld = [&](int q, u32x4n& val, uint32_t& dst) {
      const int j = c0 + CHQ * q + RPW * wave + sub;
      const int src = __shfl(kr, RPW * q + sub);
      const bool mv = j < B && src >= 0 && src != j && src < g.n_slots;  // out-of-range sources are ignored
      dst = mv ? (uint32_t)j * RB + part : kOff;
      val = __builtin_bit_cast(u32x4n, __builtin_amdgcn_raw_buffer_load_b128(
                                           src_rs, mv ? (uint32_t)src * RB + part : kOff, 0, kNt));
    };
    ld(0, x.v0, x.d0); ld(1, x.v1, x.d1); ld(2, x.v2, x.d2); ld(3, x.v3, x.d3);
    ld(4, x.v4, x.d4); ld(5, x.v5, x.d5); ld(6, x.v6, x.d6); ld(7, x.v7, x.d7);
    ld(8, x.v8, x.d8); ld(9, x.v9, x.d9); ld(10, x.v10, x.d10); ld(11, x.v11, x.d11);
    ld(12, x.v12, x.d12); ld(13, x.v13, x.d13); ld(14, x.v14, x.d14); ld(15, x.v15, x.d15);
  };
  // The chunk's loads have returned (the compiler waits for the registers the
  // empty asm reads; its memory clobber keeps the loads issued before it in
  // front), then every thread's have (the barrier).
  auto landed = [&](Buf& x) {
    asm volatile("" ::"v"(x.v0), "v"(x.v1), "v"(x.v2), "v"(x.v3), "v"(x.v4), "v"(x.v5), "v"(x.v6), "v"(x.v7),
                 "v"(x.v8), "v"(x.v9), "v"(x.v10), "v"(x.v11), "v"(x.v12), "v"(x.v13), "v"(x.v14), "v"(x.v15)
                 : "memory");
    __syncthreads();
  };
  auto store_chunk = [&](const Buf& x) {
    auto st = [&](const u32x4n& val, uint32_t dst) {
      __builtin_amdgcn_raw_buffer_store_b128(val, dst_rs, dst, 0, kNt);
    };
    st(x.v0, x.d0); st(x.v1, x.d1); st(x.v2, x.d2); st(x.v3, x.d3);
    st(x.v4, x.d4); st(x.v5, x.d5); st(x.v6, x.d6); st(x.v7, x.d7);
    st(x.v8, x.d8); st(x.v9, x.d9); st(x.v10, x.d10); st(x.v11, x.d11);
    st(x.v12, x.d12); st(x.v13, x.d13); st(x.v14, x.d14); st(x.v15, x.d15);
  };
  // Chunks past the last are loaded too (their rows are past the budget: no
  // access, nothing stored), so that no load sits behind a branch.
  Buf a, b;
  int kra = load_kr(0), krb = load_kr(1);
  load_chunk(0, kra, a);
  for (int c = 0; c < nch; c += 2) {
    kra = load_kr(c + 2);
    load_chunk(c + 1, krb, b);
    landed(a);
    store_chunk(a);
    if (c + 1 >= nch) break;
    krb = load_kr(c + 3);
    load_chunk(c + 2, kra, a);
    landed(b);
    store_chunk(b);
  }
}

}  // namespace rkv
