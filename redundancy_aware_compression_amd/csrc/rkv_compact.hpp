// In-place, order-preserving compaction of one (slice, K|V) row block,
// shared by the compaction kernel and the fused eviction-step kernel.
//
// Safety of the in-place gather: keep is ascending with keep[j] >= j, so when
// destinations are processed in ascending chunks, a chunk's writes land below
// every source of every later chunk, and its own sources are all read before
// any of its writes (loads, a full vmcnt wait, then a barrier, then stores).
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
template <typename T>
__device__ inline void compact_rows(char* base, const int32_t* __restrict__ krow, const Geom& g) {
  constexpr int RB = kHeadDim * Elem<T>::kBytes;
  constexpr int U4_ROW = RB / 16;
  constexpr int CH_ROWS = kCompactThreads * kCompactUnroll / U4_ROW;
  const int B = g.budget, tid = threadIdx.x;
  // Sixteen 16-byte loads per thread per chunk, held in named registers (an
  // array here is kept in scratch memory across the barrier by the compiler).
  static_assert(kCompactUnroll == 16, "the chunk body below is written out for 16 loads");
  for (int c0 = 0; c0 < B; c0 += CH_ROWS) {
    u32x4n v0, v1, v2, v3, v4, v5, v6, v7, v8, v9, v10, v11, v12, v13, v14, v15;
    uint32_t mvmask = 0;
    auto ld = [&](int q, u32x4n& val) {
      const int idx = q * kCompactThreads + tid;
      const int jr = c0 + idx / U4_ROW;
      const int j = min(jr, B - 1), part = idx % U4_ROW;
      const int src = krow[j];
      const bool mv = jr < B && src >= 0 && src != j && src < g.n_slots;  // out-of-range sources are ignored
      mvmask |= (uint32_t)mv << q;
      // rows that stay put load their own (in-bounds) bytes and store nothing
      val = load_nt(base + (size_t)(mv ? src : j) * RB + part * 16);
    };
    ld(0, v0); ld(1, v1); ld(2, v2); ld(3, v3); ld(4, v4); ld(5, v5); ld(6, v6); ld(7, v7);
    ld(8, v8); ld(9, v9); ld(10, v10); ld(11, v11); ld(12, v12); ld(13, v13); ld(14, v14); ld(15, v15);
    // every source of this chunk is in registers before any row is overwritten
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    auto st = [&](int q, const u32x4n& val) {
      const int idx = q * kCompactThreads + tid;
      if ((mvmask >> q) & 1u) store_nt(base + (size_t)(c0 + idx / U4_ROW) * RB + (idx % U4_ROW) * 16, val);
    };
    st(0, v0); st(1, v1); st(2, v2); st(3, v3); st(4, v4); st(5, v5); st(6, v6); st(7, v7);
    st(8, v8); st(9, v9); st(10, v10); st(11, v11); st(12, v12); st(13, v13); st(14, v14); st(15, v15);
  }
}

}  // namespace rkv
