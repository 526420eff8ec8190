// librkv C ABI: argument validation, workspace carving and kernel sequencing.
// Validation runs entirely on the host before anything is enqueued, so every
// error path leaves device memory untouched and needs no GPU.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "rkv.h"
#include "rkv_internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

rkv_status check_params(const rkv_params* p) {
  if (!p) return RKV_ERR_NULL_ARG;
  if (p->dtype != RKV_BF16 && p->dtype != RKV_F32) return RKV_ERR_BAD_PARAM;
  if (!(p->lambda >= 0.f && p->lambda <= 1.f)) return RKV_ERR_BAD_PARAM;
  if (!(p->sim_threshold >= -1.f && p->sim_threshold <= 1.f)) return RKV_ERR_BAD_PARAM;
  if (p->beta < 0) return RKV_ERR_BAD_PARAM;
  if (p->num_layers < 1 || p->num_layers > RKV_MAX_LAYERS) return RKV_ERR_BAD_SHAPE;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->group < 1) return RKV_ERR_BAD_SHAPE;
  if (p->obs_window < 1 || p->budget <= p->obs_window || p->buffer < 1) return RKV_ERR_BAD_SHAPE;
  if (p->head_dim < 1) return RKV_ERR_BAD_SHAPE;
  if ((int64_t)p->budget + p->buffer > p->capacity) return RKV_ERR_BAD_SHAPE;
  if (p->capacity > RKV_MAX_CAPACITY) return RKV_ERR_UNSUPPORTED;
  if (p->head_dim != rkv::kHeadDim) return RKV_ERR_UNSUPPORTED;
  if ((int64_t)p->group * p->obs_window > RKV_MAX_QROWS) return RKV_ERR_UNSUPPORTED;
  // slices index 1-D grids (times a few work-groups per slice) and 2-D grids' y
  const int64_t slices = (int64_t)p->num_layers * p->batch * p->num_kv_heads;
  if (slices > 65535) return RKV_ERR_UNSUPPORTED;
  return RKV_OK;
}

rkv_status check_layers(const rkv_params* p, const void* const* layers) {
  if (!layers) return RKV_ERR_NULL_ARG;
  for (int l = 0; l < p->num_layers; ++l) {
    if (!layers[l]) return RKV_ERR_NULL_ARG;
    if (!aligned16(layers[l])) return RKV_ERR_MISALIGNED;
  }
  return RKV_OK;
}

rkv::Geom make_geom(const rkv_params* p, int32_t n_slots) {
  rkv::Geom g;
  g.L = p->num_layers;
  g.batch = p->batch;
  g.H = p->num_kv_heads;
  g.G = p->group;
  g.capacity = p->capacity;
  g.budget = p->budget;
  g.alpha = p->obs_window;
  g.beta = p->beta;
  g.n_slots = n_slots;
  g.qrows = p->group * p->obs_window;
  g.lambda = p->lambda;
  g.tau = p->sim_threshold == 0.f ? 0.f : p->sim_threshold;  // -0 compares as +0: S > -0 iff S > 0
  return g;
}

rkv::LayerPtrs make_layers(const rkv_params* p, const void* const* layers) {
  rkv::LayerPtrs lp;
  memset(&lp, 0, sizeof(lp));
  for (int l = 0; l < p->num_layers; ++l) lp.p[l] = layers[l];
  return lp;
}

rkv_status hip_status(int err) {
  if (err == 0) return RKV_OK;
  g_last_hip_error = err;
  return RKV_ERR_HIP;
}

#define RKV_TRY(x)                         \
  do {                                     \
    rkv_status st_ = hip_status((x));      \
    if (st_ != RKV_OK) return st_;         \
  } while (0)

// The scoring pass: the bf16 kernel (one work-group per slice, rkv_gram.hip)
// or, for fp32 keys, the three-kernel pass of rkv_f32.hip on the workspace's
// fp32 regions.
int score(const rkv::Geom& g, int dtype, const rkv::LayerPtrs& k, const void* obs_q, const int32_t* seq_start,
          const int32_t* order, const rkv::Workspace& w, float* importance, float* rowmean, int32_t* counts,
          void* stream, const float* imp_acc) {
  if (dtype == RKV_F32)
    return rkv::launch_score_f32(g, k, obs_q, seq_start, order, w.f32_norms, w.f32_parts, importance, rowmean,
                                 counts, stream, imp_acc);
  return rkv::launch_gram(g, dtype, k, obs_q, seq_start, order, importance, rowmean, counts, stream, imp_acc);
}

// RKV_DEBUG: a non-zero integer in the environment variable at the time of
// the call turns the device precondition checks on.
bool debug_checks() {
  const char* e = getenv("RKV_DEBUG");
  return e && atoi(e) != 0;
}

// The checks of rkv_debug.hip on the step's inputs, then a sync of the
// stream and the violation bits read back: RKV_ERR_PRECONDITION when any is
// set. vl.p[0] == NULL: no values to check.
rkv_status debug_check(const rkv::Geom& g, int dtype, const rkv::LayerPtrs& kl, const rkv::LayerPtrs& vl,
                       const void* obs_q, const int32_t* seq_start, const int32_t* order, const rkv::Workspace& w,
                       void* stream) {
  RKV_TRY(rkv::launch_debug_check(g, dtype, kl, vl, obs_q, seq_start, order, w.flags, stream));
  RKV_TRY((int)hipStreamSynchronize((hipStream_t)stream));
  uint32_t bits = 0u;
  RKV_TRY((int)hipMemcpy(&bits, w.flags, sizeof(bits), hipMemcpyDeviceToHost));
  return bits ? RKV_ERR_PRECONDITION : RKV_OK;
}

}  // namespace

extern "C" {

size_t rkv_workspace_bytes(const rkv_params* p) {
  if (check_params(p) != RKV_OK) return 0;
  return rkv::carve(*p, nullptr).bytes;
}

size_t rkv_workspace_keep_offset(const rkv_params* p) {
  if (check_params(p) != RKV_OK) return (size_t)-1;
  return (size_t)(uintptr_t)rkv::carve(*p, (void*)(uintptr_t)256).keep - 256;
}

const char* rkv_status_string(rkv_status st) {
  switch (st) {
    case RKV_OK: return "RKV_OK";
    case RKV_ERR_NULL_ARG: return "RKV_ERR_NULL_ARG";
    case RKV_ERR_BAD_SHAPE: return "RKV_ERR_BAD_SHAPE";
    case RKV_ERR_BAD_PARAM: return "RKV_ERR_BAD_PARAM";
    case RKV_ERR_WORKSPACE_TOO_SMALL: return "RKV_ERR_WORKSPACE_TOO_SMALL";
    case RKV_ERR_MISALIGNED: return "RKV_ERR_MISALIGNED";
    case RKV_ERR_UNSUPPORTED: return "RKV_ERR_UNSUPPORTED";
    case RKV_ERR_HIP: return "RKV_ERR_HIP";
    case RKV_ERR_PRECONDITION: return "RKV_ERR_PRECONDITION";
  }
  return "RKV_ERR_UNKNOWN";
}

int rkv_last_hip_error(void) { return g_last_hip_error; }

rkv_status rkv_score(const rkv_params* p, const void* const* k_layers, const void* obs_q, const int32_t* seq_start,
                     int32_t n_slots, float* importance, float* redundancy, int32_t* counts, void* ws,
                     size_t ws_bytes, void* stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if ((st = check_layers(p, k_layers)) != RKV_OK) return st;
  if (!obs_q || !seq_start || !importance || !redundancy || !ws) return RKV_ERR_NULL_ARG;
  if (!aligned16(obs_q) || ((uintptr_t)ws & 255u)) return RKV_ERR_MISALIGNED;
  if (n_slots < 0 || n_slots > p->capacity) return RKV_ERR_BAD_SHAPE;
  rkv::Workspace w = rkv::carve(*p, ws);
  if (ws_bytes < w.bytes) return RKV_ERR_WORKSPACE_TOO_SMALL;
  if (n_slots <= p->budget) return RKV_OK;  // no sequence can exceed the budget
  const rkv::Geom g = make_geom(p, n_slots);
  const rkv::LayerPtrs kl = make_layers(p, k_layers);
  if (debug_checks()) {
    rkv::LayerPtrs none;
    memset(&none, 0, sizeof(none));
    if ((st = debug_check(g, p->dtype, kl, none, obs_q, seq_start, nullptr, w, stream)) != RKV_OK) return st;
  }
  int32_t* cnt = counts ? counts : w.counts;
  RKV_TRY(score(g, p->dtype, kl, obs_q, seq_start, nullptr, w, importance, w.rowmean, cnt, stream, nullptr));
  RKV_TRY(rkv::launch_redundancy(g, seq_start, cnt, w.rowmean, redundancy, stream));
  return RKV_OK;
}

rkv_status rkv_select(const rkv_params* p, const float* importance, const float* redundancy,
                      const int32_t* seq_start, int32_t n_slots, int32_t* keep, float* z_out, float* r_out,
                      void* stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if (!importance || !redundancy || !seq_start || !keep) return RKV_ERR_NULL_ARG;
  if (n_slots < p->budget || n_slots > p->capacity) return RKV_ERR_BAD_SHAPE;
  const rkv::Geom g = make_geom(p, n_slots);
  RKV_TRY(rkv::launch_select(g, importance, redundancy, nullptr, nullptr, seq_start, keep, z_out, r_out, stream));
  return RKV_OK;
}

rkv_status rkv_compact(const rkv_params* p, void* const* k_layers, void* const* v_layers, const int32_t* keep,
                       int32_t* seq_start, int32_t n_slots, void* stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if ((st = check_layers(p, (const void* const*)k_layers)) != RKV_OK) return st;
  if ((st = check_layers(p, (const void* const*)v_layers)) != RKV_OK) return st;
  if (!keep || !seq_start) return RKV_ERR_NULL_ARG;
  if (n_slots < p->budget || n_slots > p->capacity) return RKV_ERR_BAD_SHAPE;
  const rkv::Geom g = make_geom(p, n_slots);
  RKV_TRY(rkv::launch_compact(g, p->dtype, make_layers(p, (const void* const*)k_layers),
                              make_layers(p, (const void* const*)v_layers), keep, seq_start, stream));
  return RKV_OK;
}

}  // extern "C"

namespace {

// SkipKV sentence inputs of the step (see rkv_evict_step_sentences).
struct SentenceArgs {
  int32_t* sent_id;
  const float* vectors;
  const int32_t* n_sent;
  int32_t s_max, dim;
  float tau_s;
  float* penalty;
};

rkv_status check_sentences(const SentenceArgs& a) {
  if (!a.sent_id || !a.vectors || !a.n_sent || !a.penalty) return RKV_ERR_NULL_ARG;
  if (((uintptr_t)a.vectors & 15u) || ((uintptr_t)a.sent_id & 3u)) return RKV_ERR_MISALIGNED;
  if (a.s_max < 1 || a.dim < 4 || (a.dim & 3) || a.dim > rkv::kSentMaxDim) return RKV_ERR_BAD_SHAPE;
  if (!(a.tau_s >= -1.f && a.tau_s <= 1.f)) return RKV_ERR_BAD_PARAM;
  return RKV_OK;
}

// The eviction step; with `order` the hole-filling layout (gathered scoring
// loads, hole-filling compaction), else the order-preserving one; with
// `sent` SkipKV's sentence deduction and the sentence-id sidecar.
rkv_status evict_impl(const rkv_params* p, void* const* k_layers, void* const* v_layers, const void* obs_q,
                      int32_t* seq_start, int32_t* order, bool holefill, int32_t* n_slots, void* ws, size_t ws_bytes,
                      void* stream, void* const* stage_events, const SentenceArgs* sent = nullptr,
                      const float* imp_acc = nullptr, bool builtin_ws = false) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if ((st = check_layers(p, (const void* const*)k_layers)) != RKV_OK) return st;
  if ((st = check_layers(p, (const void* const*)v_layers)) != RKV_OK) return st;
  if ((!obs_q && !imp_acc) || !seq_start || !n_slots || (!ws && !builtin_ws) || (holefill && !order))
    return RKV_ERR_NULL_ARG;
  if (holefill && rkv::holefill_lds_bytes(p->budget) > rkv::kHolefillMaxLds) return RKV_ERR_UNSUPPORTED;
  if (sent && (st = check_sentences(*sent)) != RKV_OK) return st;
  if (!aligned16(obs_q) || ((uintptr_t)ws & 255u) || ((uintptr_t)order & 3u) || ((uintptr_t)imp_acc & 3u))
    return RKV_ERR_MISALIGNED;
  const int32_t ns = *n_slots;
  if (ns < 0 || ns > p->capacity) return RKV_ERR_BAD_SHAPE;
  rkv::Workspace w = rkv::carve(*p, ws);
  if (ws_bytes < w.bytes) return RKV_ERR_WORKSPACE_TOO_SMALL;
  // R-KV compresses once budget + buffer slots are full; below that, no-op.
  if (ns < p->budget + p->buffer) return RKV_OK;
  if (builtin_ws) {  // every argument is valid: only now is the device's built-in workspace looked up
    RKV_TRY(rkv::scratch_workspace(&ws));
    w = rkv::carve(*p, ws);
  }
  const rkv::Geom g = make_geom(p, ns);
  const rkv::LayerPtrs kl = make_layers(p, (const void* const*)k_layers);
  const rkv::LayerPtrs vl = make_layers(p, (const void* const*)v_layers);
  if (debug_checks() &&
      (st = debug_check(g, p->dtype, kl, vl, obs_q, seq_start, holefill ? order : nullptr, w, stream)) != RKV_OK)
    return st;
  auto mark = [&](int i) -> int {
    if (!stage_events || !stage_events[i]) return 0;
    return (int)hipEventRecord((hipEvent_t)stage_events[i], (hipStream_t)stream);
  };
  // bf16 keys in the order-preserving layout: one launch scores, selects and
  // compacts each slice (the timed variant keeps the stages apart, so that
  // each can be timed)
  if (p->dtype == RKV_BF16 && !holefill && !stage_events) {
    if (sent)
      RKV_TRY(rkv::launch_sentence_penalty(sent->vectors, sent->n_sent, p->batch, sent->s_max, sent->dim,
                                           sent->tau_s, sent->penalty, stream));
    RKV_TRY(rkv::launch_fused_step(g, p->dtype, kl, vl, obs_q, seq_start, w.importance, w.rowmean, w.counts, w.keep,
                                   stream, imp_acc, sent ? sent->penalty : nullptr, sent ? sent->sent_id : nullptr,
                                   sent ? sent->s_max : 0));
    *n_slots = p->budget;
    return RKV_OK;
  }
  RKV_TRY(mark(0));
  if (sent)
    RKV_TRY(rkv::launch_sentence_penalty(sent->vectors, sent->n_sent, p->batch, sent->s_max, sent->dim, sent->tau_s,
                                         sent->penalty, stream));
  RKV_TRY(score(g, p->dtype, kl, obs_q, seq_start, holefill ? order : nullptr, w, w.importance, w.rowmean,
                w.counts, stream, imp_acc));
  RKV_TRY(mark(1));
  RKV_TRY(rkv::launch_select(g, w.importance, nullptr, w.counts, w.rowmean, seq_start, w.keep, nullptr, nullptr,
                             stream, sent ? sent->penalty : nullptr, sent ? sent->sent_id : nullptr,
                             sent ? sent->s_max : 0));
  RKV_TRY(mark(2));
  if (holefill)
    RKV_TRY(rkv::launch_compact_holefill(g, p->dtype, kl, vl, w.keep, order, seq_start, stream));
  else
    RKV_TRY(rkv::launch_compact(g, p->dtype, kl, vl, w.keep, seq_start, stream));
  if (sent) RKV_TRY(rkv::launch_compact_ids(g, w.keep, sent->sent_id, stream));
  RKV_TRY(mark(3));
  *n_slots = p->budget;
  return RKV_OK;
}

}  // namespace

extern "C" {

rkv_status rkv_evict_step_timed(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                const void* obs_q, int32_t* seq_start, int32_t* n_slots, void* ws, size_t ws_bytes,
                                void* stream, void* const* stage_events) {
  return evict_impl(p, k_layers, v_layers, obs_q, seq_start, nullptr, false, n_slots, ws, ws_bytes, stream,
                    stage_events);
}

rkv_status rkv_evict_step(const rkv_params* p, void* const* k_layers, void* const* v_layers, const void* obs_q,
                          int32_t* seq_start, int32_t* n_slots, void* ws, size_t ws_bytes, void* stream) {
  return evict_impl(p, k_layers, v_layers, obs_q, seq_start, nullptr, false, n_slots, ws, ws_bytes, stream, nullptr);
}

rkv_status rkv_evict_step_holefill(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                   const void* obs_q, int32_t* seq_start, int32_t* order, int32_t* n_slots, void* ws,
                                   size_t ws_bytes, void* stream) {
  return evict_impl(p, k_layers, v_layers, obs_q, seq_start, order, true, n_slots, ws, ws_bytes, stream, nullptr);
}

rkv_status rkv_evict_step_holefill_timed(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                         const void* obs_q, int32_t* seq_start, int32_t* order, int32_t* n_slots,
                                         void* ws, size_t ws_bytes, void* stream, void* const* stage_events) {
  return evict_impl(p, k_layers, v_layers, obs_q, seq_start, order, true, n_slots, ws, ws_bytes, stream,
                    stage_events);
}

rkv_status rkv_compact_holefill(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                const int32_t* keep, int32_t* seq_start, int32_t* order, int32_t n_slots,
                                void* stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if ((st = check_layers(p, (const void* const*)k_layers)) != RKV_OK) return st;
  if ((st = check_layers(p, (const void* const*)v_layers)) != RKV_OK) return st;
  if (!keep || !seq_start || !order) return RKV_ERR_NULL_ARG;
  if (rkv::holefill_lds_bytes(p->budget) > rkv::kHolefillMaxLds) return RKV_ERR_UNSUPPORTED;
  if ((uintptr_t)order & 3u) return RKV_ERR_MISALIGNED;
  if (n_slots < p->budget || n_slots > p->capacity) return RKV_ERR_BAD_SHAPE;
  const rkv::Geom g = make_geom(p, n_slots);
  RKV_TRY(rkv::launch_compact_holefill(g, p->dtype, make_layers(p, (const void* const*)k_layers),
                                       make_layers(p, (const void* const*)v_layers), keep, order, seq_start, stream));
  return RKV_OK;
}

namespace {

rkv_status check_sampled(const rkv_params* p, int32_t keep_newest, int32_t top_k, float temperature) {
  if (keep_newest < 0 || keep_newest >= p->budget) return RKV_ERR_BAD_PARAM;
  if (top_k < 0) return RKV_ERR_BAD_PARAM;
  if (!(temperature > 0.f) || !(temperature < INFINITY)) return RKV_ERR_BAD_PARAM;
  return RKV_OK;
}

}  // namespace

rkv_status rkv_select_sampled(const rkv_params* p, const float* scores, const float* uniforms,
                              const int32_t* seq_start, int32_t n_slots, int32_t keep_newest, int32_t top_k,
                              float temperature, int32_t* keep, void* stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if ((st = check_sampled(p, keep_newest, top_k, temperature)) != RKV_OK) return st;
  if (!scores || !uniforms || !seq_start || !keep) return RKV_ERR_NULL_ARG;
  if (n_slots < p->budget || n_slots > p->capacity) return RKV_ERR_BAD_SHAPE;
  const rkv::Geom g = make_geom(p, n_slots);
  RKV_TRY(rkv::launch_select_sampled(g, scores, uniforms, seq_start, keep_newest, top_k, temperature, keep, stream));
  return RKV_OK;
}

rkv_status rkv_evict_step_sampled(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                  const float* scores, const float* uniforms, int32_t* seq_start, int32_t* n_slots,
                                  int32_t keep_newest, int32_t top_k, float temperature, void* ws, size_t ws_bytes,
                                  void* stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if ((st = check_sampled(p, keep_newest, top_k, temperature)) != RKV_OK) return st;
  if ((st = check_layers(p, (const void* const*)k_layers)) != RKV_OK) return st;
  if ((st = check_layers(p, (const void* const*)v_layers)) != RKV_OK) return st;
  if (!scores || !uniforms || !seq_start || !n_slots || !ws) return RKV_ERR_NULL_ARG;
  if ((uintptr_t)ws & 255u) return RKV_ERR_MISALIGNED;
  const int32_t ns = *n_slots;
  if (ns < 0 || ns > p->capacity) return RKV_ERR_BAD_SHAPE;
  rkv::Workspace w = rkv::carve(*p, ws);
  if (ws_bytes < w.bytes) return RKV_ERR_WORKSPACE_TOO_SMALL;
  if (ns < p->budget + p->buffer) return RKV_OK;  // below the trigger: no-op
  const rkv::Geom g = make_geom(p, ns);
  if (debug_checks() &&
      (st = debug_check(g, p->dtype, make_layers(p, (const void* const*)k_layers),
                        make_layers(p, (const void* const*)v_layers), nullptr, seq_start, nullptr, w, stream)) !=
          RKV_OK)
    return st;
  RKV_TRY(rkv::launch_select_sampled(g, scores, uniforms, seq_start, keep_newest, top_k, temperature, w.keep,
                                     stream));
  RKV_TRY(rkv::launch_compact(g, p->dtype, make_layers(p, (const void* const*)k_layers),
                              make_layers(p, (const void* const*)v_layers), w.keep, seq_start, stream));
  *n_slots = p->budget;
  return RKV_OK;
}

rkv_status rkv_sentence_penalty(const rkv_params* p, const float* vectors, const int32_t* n_sent, int32_t s_max,
                                int32_t dim, float tau_s, float* penalty, void* stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  int32_t dummy_id = 0;
  SentenceArgs a{&dummy_id, vectors, n_sent, s_max, dim, tau_s, penalty};
  if ((st = check_sentences(a)) != RKV_OK) return st;
  RKV_TRY(rkv::launch_sentence_penalty(vectors, n_sent, p->batch, s_max, dim, tau_s, penalty, stream));
  return RKV_OK;
}

rkv_status rkv_evict_step_sentences(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                    const void* obs_q, int32_t* seq_start, int32_t* n_slots, int32_t* sent_id,
                                    const float* vectors, const int32_t* n_sent, int32_t s_max, int32_t dim,
                                    float tau_s, float* penalty, void* ws, size_t ws_bytes, void* stream) {
  SentenceArgs a{sent_id, vectors, n_sent, s_max, dim, tau_s, penalty};
  return evict_impl(p, k_layers, v_layers, obs_q, seq_start, nullptr, false, n_slots, ws, ws_bytes, stream, nullptr,
                    &a);
}

rkv_status rkv_decode_attention(const rkv_params* p, const void* const* k_layers, const void* const* v_layers,
                                const void* q, const int32_t* seq_start, int32_t n_slots, float* out,
                                float* imp_acc, void* stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if ((st = check_layers(p, k_layers)) != RKV_OK) return st;
  if ((st = check_layers(p, v_layers)) != RKV_OK) return st;
  if (!q || !seq_start || !out) return RKV_ERR_NULL_ARG;
  if (!aligned16(q) || ((uintptr_t)out & 3u) || ((uintptr_t)imp_acc & 3u)) return RKV_ERR_MISALIGNED;
  if (n_slots < 1 || n_slots > p->capacity) return RKV_ERR_BAD_SHAPE;
  if (p->group > rkv::kDecMaxG || rkv::decode_lds_bytes(p->group, n_slots) > rkv::kDecMaxLds)
    return RKV_ERR_UNSUPPORTED;
  const rkv::Geom g = make_geom(p, n_slots);
  RKV_TRY(rkv::launch_decode(g, p->dtype, make_layers(p, k_layers), make_layers(p, v_layers), q, seq_start, out,
                             imp_acc, stream));
  return RKV_OK;
}

rkv_status rkv_evict_step_noalloc(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                  const void* obs_q, int32_t* seq_start, int32_t* n_slots, void* stream) {
  return evict_impl(p, k_layers, v_layers, obs_q, seq_start, nullptr, false, n_slots, nullptr,
                    rkv::kScratchBytes, stream, nullptr, nullptr, nullptr, true);
}

rkv_status rkv_evict_step_captured(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                   const float* imp_acc, int32_t* seq_start, int32_t* n_slots, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (!imp_acc) return RKV_ERR_NULL_ARG;
  return evict_impl(p, k_layers, v_layers, nullptr, seq_start, nullptr, false, n_slots, ws, ws_bytes, stream,
                    nullptr, nullptr, imp_acc);
}

}  // extern "C"
