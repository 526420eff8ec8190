// K5 — in-place, order-preserving compaction of the kept K/V rows.
//
// R-KV notes page (yoonschallenge.tistory.com/1236), Q&A part 2, cause 3: the
// selected KV is copied into the new cache; cause 4 lists the costs this
// avoids — re-allocation and re-arrangement of KV tensors after pruning. The
// cache is compacted where it lies: row j of [0, budget) receives row keep[j].
//
// One work-group owns one (slice, K|V) row block (compact_rows, whose
// chunk order makes the in-place gather safe); different work-groups touch
// disjoint memory.
#include "rkv_compact.hpp"

namespace rkv {

template <typename T>
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(Geom g, LayerPtrs k, LayerPtrs v,
                                                                  const int32_t* __restrict__ keep,
                                                                  int32_t* __restrict__ seq_start) {
  constexpr int RB = kHeadDim * Elem<T>::kBytes;
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = wid >> 1, kv = wid & 1;
  int l, b, h;
  slice_coords(g, slice, l, b, h);
  char* base = (char*)(kv ? v.p[l] : k.p[l]) + ((size_t)b * g.H + h) * g.capacity * (size_t)RB;
  const int32_t* krow = keep + (size_t)slice * g.budget;
  if (kv == 0 && l == 0 && h == 0 && threadIdx.x == 0) seq_start[b] = leading_unkept(krow, g.budget);
  compact_rows<T>(base, krow, g);
}

// ---------------------------------------------------------------------------
// Hole-filling compaction (order-free): the slice's tokens are virtual slots
// [s0, n_slots) in age order; virtual slot v < budget lives at physical slot
// order[v], v >= budget at v, and order[0 .. budget) is a permutation of the
// physical slots [0, budget) (entries below s0 name the free ones). After
// selection the kept tokens that already lie below the budget stay where
// they are; only the kept tokens of [budget, n_slots) move, into the
// physical slots below the budget that no kept token occupies (ascending
// movers into ascending free slots); the remaining free slots go, in
// ascending order, to the virtual slots before the new s0. The rows moved
// per slice are at most n_slots - budget, instead of about budget for the
// order-preserving compaction (R-KV notes page, Q&A part 2, causes 3 and 4:
// copying the selected KV and re-arranging the cache are the costs after
// pruning). One work-group per slice; LDS holds the keep list, the old order
// and the free list as 16-bit slots and a bitmap of occupied slots.
constexpr int kHoleThreads = 256;

// Exclusive prefix sum over the work-group (wave scans, one barrier pair);
// *total receives the sum.
__device__ inline int block_exscan_hole(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    x += lane >= o ? y : 0;
  }
  if (lane == 63) red[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kHoleThreads / 64; ++i) {
    before += i < w ? red[i] : 0;
    all += red[i];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

template <typename T>
__global__ __launch_bounds__(kHoleThreads) void holefill_kernel(Geom g, LayerPtrs k, LayerPtrs v,
                                                                const int32_t* __restrict__ keep,
                                                                int32_t* __restrict__ order,
                                                                int32_t* __restrict__ seq_start) {
  constexpr int RB = kHeadDim * Elem<T>::kBytes;
  constexpr int U4_ROW = RB / 16;
  extern __shared__ __align__(16) char hole_lds[];
  const int B = g.budget, tid = threadIdx.x;
  const int nwords = (B + 31) / 32;
  uint16_t* kl = (uint16_t*)hole_lds;  // keep list (0xFFFF: none)
  uint16_t* ol = kl + B;               // old order
  uint16_t* fl = ol + B;               // free physical slots, ascending
  uint32_t* used = (uint32_t*)(hole_lds + ((6 * (size_t)B + 15) & ~(size_t)15));
  __shared__ int red[kHoleThreads / 64];

  const int slice = xcd_remap(blockIdx.x, gridDim.x);
  int l, b, h;
  slice_coords(g, slice, l, b, h);
  const int32_t* krow = keep + (size_t)slice * B;
  int32_t* orow = order + (size_t)slice * B;

  // 1. the keep list (virtual slots, ascending after the leading -1) and the old order
  int nlead = 0, nstay = 0;
  constexpr int kLd = 8;  // keep and order entries per thread per round, loaded before use
  for (int j0 = tid; j0 < B; j0 += kLd * kHoleThreads) {
    int kvs[kLd], os[kLd];
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int j = min(j0 + u * kHoleThreads, B - 1);
      kvs[u] = krow[j];
      os[u] = orow[j];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int j = j0 + u * kHoleThreads;
      if (j < B) {
        const int kv = kvs[u], o = os[u];
        const bool valid = kv >= 0 && kv < g.n_slots;
        kl[j] = valid ? (uint16_t)kv : (uint16_t)0xFFFF;
        ol[j] = (uint16_t)(o >= 0 && o < B ? o : 0xFFFF);
        nlead += kv < 0 ? 1 : 0;
        nstay += valid && kv < B ? 1 : 0;
      }
    }
  }
  for (int w = tid; w < nwords; w += kHoleThreads) used[w] = 0u;
  int both;  // the two counts in one reduction (each below 2^16)
  block_exscan_hole((nlead << 16) | nstay, red, &both);
  nlead = both >> 16;               // new first valid virtual slot
  nstay = both & 0xFFFF;            // kept tokens already below the budget
  const int j0 = nlead + nstay;     // first mover
  const int nmov = B - j0;

  // The movers (the kept tokens past the budget, a suffix of the keep list)
  // are known now: the first pass of their row loads goes out here, so that
  // its memory latency hides behind the free-list work below. Piece idx of
  // the copy is 16 bytes of row m of K (idx < nrow) or V; sources lie at or
  // past the budget and destinations below it, so no row is both read and
  // written.
  const size_t sbase = ((size_t)b * g.H + h) * g.capacity * (size_t)RB;
  char* kb = (char*)k.p[l] + sbase;
  char* vb = (char*)v.p[l] + sbase;
  constexpr int kPass = 16;  // 16-byte copies in flight per thread
  const int nrow = nmov * U4_ROW, ncopy = 2 * nrow;
  auto piece = [&](int idx, int& m, int& part, char*& base) {
    const bool isv = idx >= nrow;
    const int r = isv ? idx - nrow : idx;
    m = r / U4_ROW;
    part = r % U4_ROW;
    base = isv ? vb : kb;
  };
  u32x4n val[kPass];
#pragma unroll
  for (int u = 0; u < kPass; ++u) {
    const int idx = u * kHoleThreads + tid;
    if (idx < ncopy) {
      int m, part;
      char* base;
      piece(idx, m, part, base);
      const int src = kl[j0 + m];
      if (src != 0xFFFF && src >= B) val[u] = load_nt(base + (size_t)src * RB + part * 16);
    }
  }
  // 2. physical slots of the kept tokens that stay
  for (int j = tid; j < B; j += kHoleThreads) {
    const int kv = kl[j];
    if (kv != 0xFFFF && kv < B && ol[kv] != 0xFFFF) atomicOr(&used[ol[kv] >> 5], 1u << (ol[kv] & 31));
  }
  __syncthreads();
  // 3. free slots, ascending: per word counts, a block scan, then the slots
  const int per = (nwords + kHoleThreads - 1) / kHoleThreads;  // words per thread
  int cnt = 0;
  for (int w = tid * per; w < min(nwords, (tid + 1) * per); ++w) {
    const uint32_t valid = w == nwords - 1 && (B & 31) ? (1u << (B & 31)) - 1u : 0xFFFFFFFFu;
    cnt += __popc(~used[w] & valid);
  }
  int nfree;
  int rank = block_exscan_hole(cnt, red, &nfree);
  for (int w = tid * per; w < min(nwords, (tid + 1) * per); ++w) {
    const uint32_t valid = w == nwords - 1 && (B & 31) ? (1u << (B & 31)) - 1u : 0xFFFFFFFFu;
    uint32_t f = ~used[w] & valid;
    while (f) {
      const int bit = __ffs(f) - 1;
      f &= f - 1;
      fl[rank++] = (uint16_t)(32 * w + bit);
    }
  }
  __syncthreads();
  // 4. the new order: stayers keep their slot, movers (the kept tokens past
  // the budget, a suffix of the keep list) take the first free slots, the
  // virtual slots before the new start the rest
  for (int j = tid; j < B; j += kHoleThreads) {
    int o;
    if (j < nlead) {
      const int r = nmov + j;
      o = r < nfree ? fl[r] : 0;
    } else if (j < j0) {
      const int kv = kl[j];
      o = kv != 0xFFFF && ol[kv] != 0xFFFF ? ol[kv] : 0;
    } else {
      const int r = j - j0;
      o = r < nfree ? fl[r] : 0;
    }
    orow[j] = o;
  }
  // 5. move the rows of K and V: the first pass's loads are in flight since
  // the keep list was read; its stores, then the further passes (loads of a
  // pass all issued before its stores)
  auto store_pass = [&](int i0) {
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int idx = i0 + u * kHoleThreads + tid;
      if (idx < ncopy) {
        int m, part;
        char* base;
        piece(idx, m, part, base);
        const int src = kl[j0 + m];
        if (m < nfree && src != 0xFFFF && src >= B) store_nt(base + (size_t)fl[m] * RB + part * 16, val[u]);
      }
    }
  };
  store_pass(0);
  for (int i0 = kPass * kHoleThreads; i0 < ncopy; i0 += kPass * kHoleThreads) {
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int idx = i0 + u * kHoleThreads + tid;
      if (idx < ncopy) {
        int m, part;
        char* base;
        piece(idx, m, part, base);
        const int src = kl[j0 + m];
        if (src != 0xFFFF && src >= B) val[u] = load_nt(base + (size_t)src * RB + part * 16);
      }
    }
    store_pass(i0);
  }
  if (l == 0 && h == 0 && tid == 0) seq_start[b] = nlead;
}

int launch_compact_holefill(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const int32_t* keep,
                            int32_t* order, int32_t* seq_start, void* stream) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const size_t lds = holefill_lds_bytes(g.budget);
  if (dtype == RKV_BF16)
    RKV_LAUNCH(holefill_kernel<bf16_t>, dim3(slices), dim3(kHoleThreads), lds, s, g, k, v, keep, order,
                       seq_start);
  else
    RKV_LAUNCH(holefill_kernel<float>, dim3(slices), dim3(kHoleThreads), lds, s, g, k, v, keep, order,
                       seq_start);
  return 0;
}

int launch_compact(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const int32_t* keep,
                   int32_t* seq_start, void* stream) {
  const int slices = g.L * g.batch * g.H;
  if (slices == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == RKV_BF16)
    RKV_LAUNCH(compact_kernel<bf16_t>, dim3(2 * slices), dim3(kCompactThreads), 0, s, g, k, v, keep,
                       seq_start);
  else
    RKV_LAUNCH(compact_kernel<float>, dim3(2 * slices), dim3(kCompactThreads), 0, s, g, k, v, keep,
                       seq_start);
  return 0;
}

}  // namespace rkv
