// Internal definitions shared by the host layer and the gfx950 kernels of
// librkv: kernel-argument blocks, workspace carving and the tiling constants.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "rkv.h"

#if defined(__HIPCC__)
#define RKV_HD __host__ __device__
#else
#define RKV_HD
#endif

namespace rkv {

constexpr int kHeadDim = 128;    // D
constexpr int kRowBlock = 64;    // Gram rows (newer tokens) per LDS stage; columns per wave
constexpr int kGramWaves = 8;    // waves per Gram work-group (one slice per work-group)
constexpr int kGroupBlocks = kGramWaves;  // 64-column blocks per column group
constexpr int kXcds = 8;         // MI355X accelerator complex dies
constexpr int kCUs = 256;        // MI355X compute units

// Geometry and method parameters common to every kernel.
struct Geom {
  int32_t L, batch, H, G, capacity, budget, alpha, beta;
  int32_t n_slots;
  int32_t qrows;   // G * alpha
  float lambda, tau;
};

struct LayerPtrs {
  const void* p[RKV_MAX_LAYERS];
};

// Column groups of one slice with N valid tokens: group g holds the
// kGroupBlocks 64-token blocks of older tokens from block g*kGroupBlocks on,
// and is paired with every row block of newer tokens from its first block to
// the end of the slice.
RKV_HD inline int gram_groups(int N) { return (N + kGroupBlocks * kRowBlock - 1) / (kGroupBlocks * kRowBlock); }
RKV_HD inline int gram_row_blocks(int N, int g) { return (N + kRowBlock - 1) / kRowBlock - g * kGroupBlocks; }

// The fp32 scoring pass (rkv_f32.hip) works in chunks of kF32Chunk keys;
// each chunk leaves kF32PartFloats floats of partial statistics: the sum of
// its unit keys (128), then per query row m the (max, sum of exp) of its
// causal logits at 128 + 2 m.
constexpr int kF32Chunk = 32;
constexpr int kF32PartFloats = kHeadDim + 2 * RKV_MAX_QROWS;
RKV_HD inline int f32_chunks(int n) { return (n + kF32Chunk - 1) / kF32Chunk; }

// Workspace regions, each 256-byte aligned, sized for n_slots = capacity.
struct Workspace {
  float* rowmean;     // [slices][n_slots]
  int32_t* counts;    // [slices][n_slots]
  float* importance;  // [slices][n_slots]
  int32_t* keep;      // [slices][budget]
  uint32_t* flags;    // 64 words: the RKV_DEBUG checks' violation bits (word 0)
  float* f32_norms;   // fp32 keys only: [slices][n_slots] key norms
  float* f32_parts;   // fp32 keys only: [slices][f32_chunks(capacity)][kF32PartFloats]
  size_t bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Workspace carve(const rkv_params& p, void* base) {
  const size_t slices = (size_t)p.num_layers * p.batch * p.num_kv_heads;
  const size_t cap = (size_t)p.capacity;
  Workspace w;
  size_t off = 0;
  char* b = (char*)base;
  auto take = [&](size_t bytes) {
    char* ptr = b ? b + off : nullptr;
    off += align256(bytes);
    return ptr;
  };
  w.rowmean = (float*)take(slices * cap * 4);
  w.counts = (int32_t*)take(slices * cap * 4);
  w.importance = (float*)take(slices * cap * 4);
  w.keep = (int32_t*)take(slices * (size_t)p.budget * 4);
  w.flags = (uint32_t*)take(256);
  w.f32_norms = w.f32_parts = nullptr;
  if (p.dtype == RKV_F32) {
    w.f32_norms = (float*)take(slices * cap * 4);
    w.f32_parts = (float*)take(slices * (size_t)f32_chunks((int)cap) * kF32PartFloats * 4);
  }
  w.bytes = off;
  return w;
}

// Kernel launchers (one translation unit each). They return the hipError_t
// of the launch as an int (0 = success).
// With imp_acc (and no order) the importance comes from captured decode
// attention weights instead of obs_q.
int launch_gram(const Geom& g, int dtype, const LayerPtrs& k, const void* obs_q, const int32_t* seq_start,
                const int32_t* order, float* importance, float* rowmean, int32_t* counts, void* stream,
                const float* imp_acc = nullptr);
// The scoring pass for fp32 keys (rkv_f32.hip): statistics per chunk of
// keys, similar-pair counts per 32x32 tile of the upper triangle, then row
// means and importance per token. Same inputs and outputs as launch_gram
// (counts are accumulated: the first kernel clears them); norms and parts
// are the workspace's fp32 regions.
int launch_score_f32(const Geom& g, const LayerPtrs& k, const void* obs_q, const int32_t* seq_start,
                     const int32_t* order, float* norms, float* parts, float* importance, float* rowmean,
                     int32_t* counts, void* stream, const float* imp_acc);
int launch_redundancy(const Geom& g, const int32_t* seq_start, const int32_t* counts, const float* rowmean,
                      float* redundancy, void* stream);
int launch_select_sampled(const Geom& g, const float* scores, const float* uniforms, const int32_t* seq_start,
                          int keep_newest, int top_k, float temperature, int32_t* keep, void* stream);
int launch_select(const Geom& g, const float* importance, const float* redundancy, const int32_t* counts,
                  const float* rowmean, const int32_t* seq_start, int32_t* keep, float* z_out, float* r_out,
                  void* stream, const float* sent_pen = nullptr, const int32_t* sent_id = nullptr, int s_max = 0);
int launch_sentence_penalty(const float* vectors, const int32_t* n_sent, int batch, int s_max, int dim, float tau_s,
                            float* penalty, void* stream);
int launch_compact_ids(const Geom& g, const int32_t* keep, int32_t* ids, void* stream);
constexpr int kSentMaxDim = 8192;
// Decode attention with importance capture (rkv_decode.hip): query heads per
// KV head up to kDecMaxG; dynamic LDS of decode_lds_bytes(G, n_slots) bytes.
int launch_decode(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const void* q,
                  const int32_t* seq_start, float* out, float* acc, void* stream);
constexpr int kDecMaxWaves = 8;
// the weights of every query head over max(n_slots, kDecMaxWaves * 128) rows, fp32
inline size_t decode_lds_bytes(int group, int n_slots) {
  const int rows = n_slots > kDecMaxWaves * kHeadDim ? n_slots : kDecMaxWaves * kHeadDim;
  return (size_t)group * rows * 4;
}
constexpr int kDecMaxG = 8;
constexpr size_t kDecMaxLds = 160 * 1024 - 1024;
// dynamic LDS of the hole-filling compaction; launches keep it within 64 KB
// three uint16 tables of budget entries (16-byte aligned) and one bit per row
inline size_t holefill_lds_bytes(int budget) {
  return ((6 * (size_t)budget + 15) & ~(size_t)15) + 4 * (size_t)((budget + 31) / 32);
}
constexpr size_t kHolefillMaxLds = 65536 - 2048;
int launch_compact_holefill(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const int32_t* keep,
                            int32_t* order, int32_t* seq_start, void* stream);
int launch_compact(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const int32_t* keep,
                   int32_t* seq_start, void* stream);
// The whole order-preserving step for bf16 keys in one scoring launch
// (rkv_gram.hip): each slice's work-group scores it, selects (keep) and
// compacts its K and V rows; a second launch then writes seq_start. Same
// results as launch_gram + launch_select (counts and row means) +
// launch_compact (+ launch_compact_ids with sent_id: the sentence penalties,
// computed before, enter the selection). Needs capacity <= RKV_MAX_CAPACITY.
int launch_fused_step(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const void* obs_q,
                      int32_t* seq_start, float* importance, float* rowmean, int32_t* counts, int32_t* keep,
                      void* stream, const float* imp_acc, const float* sent_pen = nullptr, int32_t* sent_id = nullptr,
                      int s_max = 0);

// RKV_DEBUG device checks (rkv_debug.hip): clears flags[0], then ORs into
// it kDbgSeqStart when some seq_start[b] lies outside [0, n_slots],
// kDbgKV when a key or value element of a valid slot is not finite, kDbgQuery
// when an element of obs_q (if given) is not finite, kDbgOrder when order (if
// given) is not a permutation of [0, budget) for some slice.
constexpr uint32_t kDbgSeqStart = 1, kDbgKV = 2, kDbgQuery = 4, kDbgOrder = 8;
int launch_debug_check(const Geom& g, int dtype, const LayerPtrs& k, const LayerPtrs& v, const void* obs_q,
                       const int32_t* seq_start, const int32_t* order, uint32_t* flags, void* stream);

// The built-in workspace of rkv_evict_step_noalloc (rkv_scratch.hip): a
// device array of kScratchBytes per GPU; *ws receives its address on the
// current device (looked up once per device). Returns a hipError_t.
constexpr size_t kScratchBytes = (size_t)RKV_NOALLOC_WORKSPACE_BYTES;
int scratch_workspace(void** ws);

}  // namespace rkv
