/*
 * librkv — decode-time R-KV KV-cache eviction on AMD Instinct MI355X (gfx950).
 *
 * R-KV (redundancy-aware KV-cache compression for reasoning models) keeps a
 * fixed-budget KV cache during decoding. Every time budget + buffer slots are
 * full it keeps the newest observation tokens, scores every other cached
 * token by importance (observation-query attention, max-pooled over the
 * query heads of a GQA group) and by redundancy (cosine similarity of its key
 * to the other keys of the same head, with the most recent similar tokens
 * protected), combines the two and keeps the top tokens up to the budget.
 * Source: R-KV notes page (yoonschallenge.tistory.com/1236), opening notes,
 * summary table rows "decoding-time compression", "importance computation",
 * "redundancy computation", "final selection criterion", and Q&A part 2,
 * cause 3 (the per-128-token compression work).
 *
 * Readings where the page is silent (stated, not printed on the page):
 *   Z_i = lambda*I_i - (1-lambda)*R_i with R = softmax of the redundancy over
 *   the candidates; "similar" means cosine > sim_threshold; token i is
 *   protected (redundancy 0) iff fewer than beta newer tokens are similar to
 *   it; otherwise its redundancy is its mean cosine to the other N-1 valid
 *   tokens; the budget includes the observation window; equal scores go to
 *   the newer token; each (layer, sequence, KV head) selects independently.
 *
 * CONVENTIONS (every entry point)
 *   Memory. Every pointer is a DEVICE pointer unless marked HOST. The caller
 *   owns all memory; the library never allocates or frees device memory and
 *   keeps no state between calls except a thread-local last HIP error and
 *   the built-in workspace of rkv_evict_step_noalloc (a device array in the
 *   code object, not an allocation).
 *   Layout. Per-layer caches K and V are [batch][num_kv_heads][capacity]
 *   [head_dim] rows, contiguous (row stride head_dim elements), 16-byte
 *   aligned. Sequence b holds N_b = n_slots - seq_start[b] valid tokens in
 *   slots [seq_start[b], n_slots) (left padding); padding slots are never
 *   read. obs_q is [num_layers][batch][num_kv_heads*group][obs_window]
 *   [head_dim], same element type; query head hq belongs to KV head
 *   hq / group; row t of a head is the query of token N_b - obs_window + t.
 *   Score arrays are float32 [num_layers][batch][num_kv_heads][n_slots]
 *   indexed by slot; keep is int32 [num_layers][batch][num_kv_heads][budget].
 *   Streams. `stream` is a hipStream_t (NULL = the null stream). Work is
 *   enqueued asynchronously; no entry point synchronises the host.
 *   Errors. Arguments are validated on the host before anything is
 *   enqueued; on any error nothing is launched and nothing is written.
 *   A failed launch returns RKV_ERR_HIP (see rkv_last_hip_error). Device
 *   data preconditions (0 <= seq_start[b] <= n_slots, finite values in valid
 *   slots) cannot be checked without a host sync: the kernels clamp
 *   seq_start into range so a violation never addresses memory outside the
 *   caller's buffers, but the result is then unspecified. No entry point
 *   prints, aborts or throws.
 *   Debug checks. When the environment variable RKV_DEBUG holds a non-zero
 *   integer at the time of a call, rkv_score and every rkv_evict_step*
 *   entry point that would launch work first check those preconditions on
 *   the device: every seq_start[b] within [0, n_slots]; every key and value
 *   element of the valid slots and every observation-query element finite
 *   (those the call reads); with the hole-filling layout, each slice's order
 *   a permutation of [0, budget). They then synchronise `stream` and, on a
 *   violation, return RKV_ERR_PRECONDITION with nothing else launched and
 *   nothing written but the workspace. Off by default; benchmarks leave it
 *   off.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RKV_OK = 0,
  RKV_ERR_NULL_ARG = 1,            /* a required pointer is NULL                      */
  RKV_ERR_BAD_SHAPE = 2,           /* sizes out of range or inconsistent              */
  RKV_ERR_BAD_PARAM = 3,           /* lambda, sim_threshold, beta or dtype invalid    */
  RKV_ERR_WORKSPACE_TOO_SMALL = 4, /* ws_bytes < rkv_workspace_bytes(p)               */
  RKV_ERR_MISALIGNED = 5,          /* a tensor pointer is not 16-byte aligned         */
  RKV_ERR_UNSUPPORTED = 6,         /* valid but not implemented (e.g. head_dim != 128) */
  RKV_ERR_HIP = 7,                 /* a HIP launch failed                             */
  RKV_ERR_PRECONDITION = 8         /* RKV_DEBUG: a device-data precondition failed    */
} rkv_status;

typedef enum { RKV_BF16 = 0, RKV_F32 = 1 } rkv_dtype;

#define RKV_MAX_LAYERS 128     /* per-layer pointers travel by value in kernel arguments */
#define RKV_MAX_CAPACITY 16384 /* slots per (sequence, head) row block                   */
#define RKV_MAX_QROWS 64       /* group * obs_window                                     */

typedef struct {
  int32_t num_layers;   /* L, 1..RKV_MAX_LAYERS                                     */
  int32_t batch;        /* sequences per layer tensor, >= 1                         */
  int32_t num_kv_heads; /* KV heads, >= 1                                           */
  int32_t group;        /* query heads per KV head (GQA group), >= 1                */
  int32_t head_dim;     /* D; 128 is the only supported value                       */
  int32_t capacity;     /* slots per (sequence, head); >= budget + buffer           */
  int32_t budget;       /* B: tokens kept per (sequence, head), window included     */
  int32_t buffer;       /* new tokens between evictions (R-KV default 128), >= 1    */
  int32_t obs_window;   /* alpha: observation tokens (R-KV default 8), 1..budget-1  */
  int32_t beta;         /* protection count, >= 0                                   */
  float lambda;         /* importance weight in [0, 1] (R-KV best: 0.1)             */
  float sim_threshold;  /* tau in [-1, 1]                                           */
  int32_t dtype;        /* rkv_dtype of K, V and obs_q                              */
} rkv_params;

/* Bytes of device workspace rkv_score and rkv_evict_step need for p (sized
 * for n_slots = capacity); 0 if p is invalid. Any 256-byte-aligned buffer of
 * at least this size works; its content need not be initialised and is
 * clobbered. */
size_t rkv_workspace_bytes(const rkv_params* p);

/* Byte offset, inside the workspace, of the keep lists rkv_evict_step writes:
 * int32 [num_layers][batch][num_kv_heads][budget], the same convention as
 * rkv_select's keep (source slot of each destination slot, ascending,
 * right-aligned, -1 before the kept entries). They stay valid after the step
 * until the workspace is used again; a caller that keeps per-token metadata
 * beside the cache (positions, token ids) remaps it with them (R-KV notes
 * page, Q&A part 2, cause 3: selection indices drive the copy of the kept
 * entries). Returns (size_t)-1 if p is invalid. */
size_t rkv_workspace_keep_offset(const rkv_params* p);

/*
 * Importance and redundancy of every valid token of every (layer, sequence,
 * KV head) whose sequence has outgrown the budget (N_b > budget); other
 * sequences' entries are left unchanged. Source: R-KV notes page, summary
 * table row "importance computation" (the attention the observation tokens
 * pay each cached token, max over the query heads that share a KV head) and
 * row "redundancy computation" (cosine similarity of a token's key to the
 * other keys of its head, the most recent similar tokens protected); Q&A part
 * 2, cause 3 (key normalisation and the all-pairs cosine of each round).
 *   k_layers   HOST array of num_layers device pointers to K caches (read only)
 *   obs_q      observation queries (read only)
 *   seq_start  [batch] int32 first valid slot per sequence (read only)
 *   n_slots    slots in use, budget < n_slots <= capacity is the useful range,
 *              0 <= n_slots <= capacity is accepted
 *   importance out: I_j = max over the group's query heads of the mean over
 *              the obs_window queries of the causal softmax attention weight
 *              on key j (scale 1/sqrt(head_dim))
 *   redundancy out: rbar_j = 0 if protected, else mean cosine of key j to the
 *              other N_b - 1 valid keys
 *   counts     out, nullable: int32 c_j = #{ newer valid tokens with cosine >
 *              sim_threshold }, the quantity the protection rule tests
 *              (token j is protected iff c_j < beta). Not one of the method's
 *              outputs: it is exposed so that callers and tests can see why a
 *              token is or is not protected; NULL uses the workspace.
 *   ws, ws_bytes  workspace (see rkv_workspace_bytes)
 */
rkv_status rkv_score(const rkv_params* p, const void* const* k_layers, const void* obs_q, const int32_t* seq_start,
                     int32_t n_slots, float* importance, float* redundancy, int32_t* counts, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Selection from given scores (R-KV notes page, summary table row "final
 * selection criterion": importance raises a token's score, redundancy lowers
 * it, lambda = 0.1 works best; opening notes: the observation tokens are
 * kept and the top-scoring others fill the budget). For each (layer,
 * sequence, KV head) with N_b > budget: R = softmax of redundancy over the
 * candidates (the N_b - obs_window oldest valid tokens), Z = lambda*I -
 * (1-lambda)*R, the
 * budget - obs_window candidates with the largest Z (equal Z: the later slot
 * wins) plus the obs_window newest tokens are kept. With N_b <= budget every
 * valid token is kept. keep[j] receives the source slot of destination slot
 * j in ascending order, right-aligned: entries [0, budget - kept) are -1.
 * keep[j] >= j always holds.
 *   importance, redundancy  score arrays (read only)
 *   seq_start  read only; budget <= n_slots <= capacity
 *   keep       out
 *   z_out, r_out  out, nullable: Z and R at candidate slots of evicting
 *              sequences (other entries unchanged)
 */
rkv_status rkv_select(const rkv_params* p, const float* importance, const float* redundancy,
                      const int32_t* seq_start, int32_t n_slots, int32_t* keep, float* z_out, float* r_out,
                      void* stream);

/*
 * In-place, order-preserving compaction (R-KV notes page, Q&A part 2, cause
 * 3: the selected entries are copied into the compressed cache; cause 4:
 * allocation and re-allocation cost, avoided here by moving rows within the
 * caller's cache): for every (layer, sequence, KV
 * head) row j of K and V in [0, budget) with keep[j] >= 0 receives the bytes
 * of row keep[j]; then seq_start[b] = number of -1 entries of the sequence's
 * keep rows. Rows with keep[j] = -1 and rows >= budget are left as they are.
 *   k_layers, v_layers  HOST arrays of num_layers device pointers (modified)
 *   keep       as produced by rkv_select (ascending, keep[j] >= j required)
 *   seq_start  in/out; budget <= n_slots <= capacity
 */
rkv_status rkv_compact(const rkv_params* p, void* const* k_layers, void* const* v_layers, const int32_t* keep,
                       int32_t* seq_start, int32_t n_slots, void* stream);

/*
 * One decode-time eviction step over all layers, sequences and KV heads
 * (R-KV notes page, opening notes and summary table row "decoding-time
 * compression": once budget + buffer tokens are cached, the cache is
 * compressed back to the budget; Q&A part 2, cause 3: scoring, selection and
 * copy of one such round).
 * If *n_slots < budget + buffer nothing is launched or written (RKV_OK).
 * Otherwise scoring, selection and compaction run on `stream` and *n_slots
 * becomes budget; afterwards sequence b holds min(N_b, budget) tokens in
 * slots [seq_start[b], budget), in their original order. With bf16 keys the
 * three stages run as one launch (each slice's work-group scores, selects
 * and compacts it) followed by a small kernel that writes seq_start; the
 * results are bit-identical to the staged kernels of rkv_evict_step_timed.
 *   k_layers, v_layers  HOST arrays of device pointers (modified in place)
 *   obs_q      observation queries (read only)
 *   seq_start  in/out
 *   n_slots    HOST in/out
 *   ws, ws_bytes  workspace (see rkv_workspace_bytes)
 */
rkv_status rkv_evict_step(const rkv_params* p, void* const* k_layers, void* const* v_layers, const void* obs_q,
                          int32_t* seq_start, int32_t* n_slots, void* ws, size_t ws_bytes, void* stream);

/*
 * rkv_evict_step with per-stage timing events, for benchmarks and profilers.
 * stage_events: HOST array of 4 hipEvent_t created by the caller (NULL
 * entries are skipped). Event s is recorded on `stream` right before stage s
 * is enqueued — 0 scoring (key statistics, Gram, importance and row mean in
 * one kernel), 1 selection, 2 compaction — and event 3 after the last one.
 * The stages always run as separate kernels here (rkv_evict_step fuses them
 * for bf16 keys), with the same results. On the no-op path no event is
 * recorded. Everything else is exactly rkv_evict_step.
 */
rkv_status rkv_evict_step_timed(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                const void* obs_q, int32_t* seq_start, int32_t* n_slots, void* ws, size_t ws_bytes,
                                void* stream, void* const* stage_events);

/*
 * Hole-filling layout (order-free compaction with an order sidecar). The
 * pages name the copy of the kept entries and the re-arrangement of the cache
 * as costs of pruning (R-KV notes page, Q&A part 2, causes 3 and 4); in this
 * layout an eviction moves only the kept tokens that arrived since the last
 * one. Sequence b's valid tokens are the virtual slots [seq_start[b],
 * n_slots) in age order. Virtual slot v < budget is stored at physical slot
 * order[slice][v], v >= budget at physical slot v (new tokens are appended
 * there in order). order is int32 [num_layers][batch][num_kv_heads][budget]
 * and each slice's row is a permutation of [0, budget); its entries below
 * seq_start[b] name the free physical slots. The identity permutation turns
 * a cache laid out for rkv_evict_step into this layout.
 *
 * rkv_evict_step_holefill: the eviction of rkv_evict_step (same trigger,
 * scores and kept set, computed on the virtual order) with the compaction
 * replaced: kept tokens below the budget stay in their physical slots; the
 * kept tokens of [budget, n_slots) move, in ascending virtual order, into
 * the ascending physical slots below the budget that no kept token occupies;
 * the remaining free slots go, ascending, to the virtual slots before the new
 * seq_start. order and seq_start are rewritten (in/out), *n_slots becomes
 * budget. At most n_slots - budget rows of K and of V move per slice. Errors
 * as rkv_evict_step, plus RKV_ERR_NULL_ARG for a NULL order,
 * RKV_ERR_MISALIGNED for an order not 4-byte aligned and
 * RKV_ERR_UNSUPPORTED for a budget above 10,000 (the compaction's LDS). An order row that is
 * not a permutation gives unspecified slots but no access outside the
 * slice's rows.
 */
rkv_status rkv_evict_step_holefill(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                   const void* obs_q, int32_t* seq_start, int32_t* order, int32_t* n_slots, void* ws,
                                   size_t ws_bytes, void* stream);

/* rkv_evict_step_holefill with the four stage events of rkv_evict_step_timed. */
rkv_status rkv_evict_step_holefill_timed(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                         const void* obs_q, int32_t* seq_start, int32_t* order, int32_t* n_slots,
                                         void* ws, size_t ws_bytes, void* stream, void* const* stage_events);

/* The compaction of rkv_evict_step_holefill from a given keep list (the
 * layout of rkv_select's keep: virtual slots, ascending, right-aligned, -1
 * before the kept entries). keep is read only; order and seq_start are
 * rewritten. budget <= n_slots <= capacity. */
rkv_status rkv_compact_holefill(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                const int32_t* keep, int32_t* seq_start, int32_t* order, int32_t n_slots,
                                void* stream);

/*
 * Sampled selection (ForesightKV explainer, technical summary: eviction is
 * triggered at budget + L; the newest L tokens stay and the rest is
 * compressed to budget - L from a scoring model's per-token importance, the
 * eviction decision being a Top-K followed by multinomial sampling). The
 * scores are the caller's (the learned scoring model is not part of this
 * library). Per (layer, sequence, KV head) with N_b > budget: the newest
 * keep_newest valid tokens are kept; of the other (candidate) tokens the
 * top_k by score are retained first (equal scores: the later slot; top_k is
 * raised to budget - keep_newest and capped at the candidate count), and
 * budget - keep_newest of those are drawn without replacement with
 * probabilities proportional to exp(score / temperature), in the
 * Gumbel-top-k form: the largest score / temperature - log(-log u), u the
 * caller's uniform for the slot. With N_b <= budget every valid token is
 * kept.
 *   scores, uniforms  float32 [num_layers][batch][num_kv_heads][n_slots],
 *                     read at the valid slots; uniforms strictly in (0, 1)
 *   keep_newest       L, 0 <= L < budget
 *   top_k             >= 0; temperature > 0 and finite
 *   keep              out, the layout of rkv_select's keep
 * Errors as rkv_select, plus RKV_ERR_BAD_PARAM for keep_newest, top_k or
 * temperature out of range.
 */
rkv_status rkv_select_sampled(const rkv_params* p, const float* scores, const float* uniforms,
                              const int32_t* seq_start, int32_t n_slots, int32_t keep_newest, int32_t top_k,
                              float temperature, int32_t* keep, void* stream);

/* The eviction step with the sampled selection: the trigger of
 * rkv_evict_step (n_slots >= budget + buffer, else a no-op), then
 * rkv_select_sampled into the workspace's keep lists
 * (rkv_workspace_keep_offset) and the order-preserving compaction of
 * rkv_compact. *n_slots becomes budget. */
rkv_status rkv_evict_step_sampled(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                  const float* scores, const float* uniforms, int32_t* seq_start, int32_t* n_slots,
                                  int32_t keep_newest, int32_t top_k, float temperature, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * Sentence-level redundancy (SkipKV notes page, summary table rows
 * "sentence-level KV storage skipping", "final eviction score" and "cache
 * range monitoring"). A sentence is represented by the mean of its tokens'
 * last-layer hidden states (the caller's vectors); when a later sentence's
 * cosine with an earlier one exceeds tau_s, the earlier one is redundant.
 * rkv_sentence_penalty: penalty[b][i] = the largest cosine of sentence i of
 * sequence b with a later sentence j < n_sent[b] when it exceeds tau_s, else
 * 0 (a zero vector is similar to nothing); entries i >= n_sent[b] are 0.
 *   vectors  float32 [batch][s_max][dim], 16-byte aligned, dim a multiple of
 *            4 and at most 8192
 *   n_sent   int32 [batch] (device), sentences per sequence, clamped to s_max
 *   penalty  out, float32 [batch][s_max]
 * Errors: RKV_ERR_NULL_ARG, RKV_ERR_MISALIGNED, RKV_ERR_BAD_SHAPE (s_max,
 * dim), RKV_ERR_BAD_PARAM (tau_s outside [-1, 1]), and those of the params.
 */
rkv_status rkv_sentence_penalty(const rkv_params* p, const float* vectors, const int32_t* n_sent, int32_t s_max,
                                int32_t dim, float tau_s, float* penalty, void* stream);

/*
 * rkv_evict_step with SkipKV's sentence deduction: the sentence penalties
 * (rkv_sentence_penalty, into the caller's penalty buffer) are subtracted
 * from Z of each candidate, by the sentence of its slot, so that tokens of
 * redundant sentences go before ordinary ones; the kept count stays the
 * token budget. sent_id: int32 [num_layers][batch][num_kv_heads][capacity],
 * the sentence index of each slot's token (-1 or >= s_max: none), in/out:
 * the compaction moves it with the K/V rows (entries of the slots before the
 * new seq_start become -1), which keeps the sentence map of the cache in
 * step with its contents. Errors: those of rkv_evict_step and
 * rkv_sentence_penalty, RKV_ERR_MISALIGNED for sent_id not 4-byte aligned.
 */
rkv_status rkv_evict_step_sentences(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                    const void* obs_q, int32_t* seq_start, int32_t* n_slots, int32_t* sent_id,
                                    const float* vectors, const int32_t* n_sent, int32_t s_max, int32_t dim,
                                    float tau_s, float* penalty, void* ws, size_t ws_bytes, void* stream);

/*
 * Decode attention with importance capture. R-KV's importance is the
 * attention that the newest obs_window queries pay each cached token (R-KV
 * notes page, summary table row "importance computation"); those rows are
 * what the decode steps compute anyway, and the notes name fusing attention,
 * importance scoring and eviction into one kernel as a way to cut the cost
 * of compression (Q&A part 2, cause 4).
 *
 * rkv_decode_attention: the newest token of every sequence attends to the
 * sequence's valid slots [seq_start[b], n_slots), its own K/V row (slot
 * n_slots - 1) included: for each query head, w = softmax over those slots
 * of q.k / sqrt(head_dim) and out = sum_j w_j v_j.
 *   k_layers, v_layers  HOST [num_layers] device pointers, the cache layout
 *                       of rkv_evict_step (16-byte aligned)
 *   q        [num_layers][batch][num_kv_heads * group][head_dim], cache dtype,
 *            16-byte aligned (query head hq belongs to KV head hq / group)
 *   out      out, float32 [num_layers][batch][num_kv_heads * group][head_dim];
 *            0 for a sequence with no valid slot
 *   imp_acc  NULL, or float32 [num_layers][batch][num_kv_heads][group][capacity]
 *            (in/out): w is ADDED at the slot of each key. Zero it before the
 *            first of the obs_window decode steps that precede an eviction
 *            (and after every eviction, whose compaction moves the slots), and
 *            pass it on those steps only; rkv_evict_step_captured then reads it.
 * Errors: those of the params and layers, RKV_ERR_NULL_ARG, RKV_ERR_MISALIGNED,
 * RKV_ERR_BAD_SHAPE (n_slots outside [1, capacity]), RKV_ERR_UNSUPPORTED
 * (group > 8, or group * max(n_slots, 1024) * 4 bytes of weights above 159 KiB).
 */
rkv_status rkv_decode_attention(const rkv_params* p, const void* const* k_layers, const void* const* v_layers,
                                const void* q, const int32_t* seq_start, int32_t n_slots, float* out,
                                float* imp_acc, void* stream);

/*
 * rkv_evict_step with the importance taken from imp_acc (filled by
 * rkv_decode_attention over the obs_window decode steps before the trigger):
 * I = max over the group of imp_acc / obs_window, which equals the importance
 * that rkv_evict_step computes from those steps' queries. The queries are not
 * read. Everything else (redundancy, selection, compaction, n_slots and
 * seq_start updates, no-op below budget + buffer) is rkv_evict_step's.
 * Errors: those of rkv_evict_step; RKV_ERR_NULL_ARG for imp_acc NULL,
 * RKV_ERR_MISALIGNED for imp_acc not 4-byte aligned.
 */
rkv_status rkv_evict_step_captured(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                   const float* imp_acc, int32_t* seq_start, int32_t* n_slots, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * rkv_evict_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Exactly rkv_evict_step (same trigger, kernels, results, n_slots and
 * seq_start updates) with no ws argument: the workspace is a device array of
 * RKV_NOALLOC_WORKSPACE_BYTES built into the library, which every GPU the
 * library runs on holds until the process ends. The call allocates nothing
 * (no hipMalloc, no allocating library routine); its first call on a device
 * looks up that device's copy of the array.
 *   Limit: parameters with rkv_workspace_bytes(p) > RKV_NOALLOC_WORKSPACE_BYTES
 *   are rejected with RKV_ERR_WORKSPACE_TOO_SMALL (nothing launched).
 *   Sharing: every call on one GPU uses that GPU's one array, and it keeps the
 *   last call's contents (nothing in it needs to start at zero). Calls that
 *   overlap on one GPU (other threads, other streams without ordering between
 *   them) race on it: order them, or use rkv_evict_step with a workspace each.
 * Errors: those of rkv_evict_step (without the workspace ones), plus
 * RKV_ERR_HIP when the array's address cannot be obtained on the device.
 */
#define RKV_NOALLOC_WORKSPACE_BYTES (32u << 20)
rkv_status rkv_evict_step_noalloc(const rkv_params* p, void* const* k_layers, void* const* v_layers,
                                  const void* obs_q, int32_t* seq_start, int32_t* n_slots, void* stream);

/* Static string naming a status. */
const char* rkv_status_string(rkv_status st);

/* hipError_t of the last failed launch on this thread (0 if none). */
int rkv_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RKV_H */
