/*
 * CPU oracle of the R-KV decode-time eviction step — TEST INFRASTRUCTURE.
 *
 * Plain, slow, single-threaded C++ in double precision. Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg use it; the HIP library
 * never links, loads or calls it, and it shares no code with that library.
 *
 * Sources (the R-KV pages):
 *   [RKV] R-KV notes page, yoonschallenge.tistory.com/1236 (NeurIPS 2025
 *         poster): opening notes, summary table, Q&A part 2 ("why did time
 *         drop less than expected"), cause 3 (per-128-token compression work)
 *         and cause 4 (attention, importance scoring and eviction fused).
 *   [SKV] SkipKV notes page, yoonschallenge.tistory.com/1230: summary table
 *         rows "sentence-level KV storage skipping" and "final eviction score".
 *   [FKV] ForesightKV explainer, gist.science/ko/paper/2602.03203: technical
 *         summary (the eviction trigger and the Top-K + multinomial draw).
 * Where the pages are silent (the combination formula, the protection rule,
 * tie order, padding) the readings below are stated at the point of use.
 *
 * Parity pins: every function is pinned by the CPU tests against hand-derived
 * closed forms, textbook special cases, library routines, invariants and brute
 * force. Parity unpinned by the pages themselves: they print no example, so
 * the readings they leave open (the combination formula, the protection rule,
 * the sentence penalty's form, the sampled draw's parameters, the free-row
 * order of the hole-filling layout) are pinned to those readings, not to
 * values the pages give.
 */
#ifndef RKV_ORACLE_H
#define RKV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_BF16 0
#define ORC_F32 1

/* One slice = one (layer, sequence, KV head). */
typedef struct {
  int32_t n;          /* valid tokens N of the slice                       */
  int32_t head_dim;   /* D                                                 */
  int32_t group;      /* G query heads per KV head                         */
  int32_t obs_window; /* alpha, observation tokens kept unconditionally    */
  int32_t budget;     /* B, kept tokens after eviction (window included)   */
  int32_t beta;       /* protection count                                  */
  double lambda;      /* weight of importance in Z = lambda*I - (1-lambda)*R */
  double tau;         /* similarity threshold: "similar" means S_ij > tau  */
  double amb_eps;     /* |S_ij - tau| <= amb_eps flags row min(i,j) as ambiguous */
} orc_slice_params;

/* Outputs of orc_slice; every pointer is nullable, arrays have N entries
 * except keep (min(N, B) entries). */
typedef struct {
  double* importance; /* I_j for every valid j                              */
  double* rowmean;    /* (1/(N-1)) * sum_{j != i} S_ij                      */
  int32_t* counts;    /* c_i = #{ j > i : S_ij > tau }                      */
  double* rbar;       /* 0 if c_i < beta, else rowmean_i                    */
  double* R;          /* softmax of rbar over the candidates, 0 elsewhere   */
  double* Z;          /* lambda*I - (1-lambda)*R over candidates, 0 elsewhere */
  int32_t* ambiguous; /* 1 where a pair (i, j>i) sits within amb_eps of tau  */
  int32_t* keep;      /* kept positions (0-based within the slice), ascending */
} orc_slice_out;

/*
 * Scores and selects one slice. keys: N rows of D values; queries: G*alpha
 * rows of D values (query head g, observation token t at row g*alpha + t;
 * token t sits at position N - alpha + t). dtype ORC_BF16 (uint16 bits) or
 * ORC_F32. When N <= B every token is kept and no score is computed.
 * Returns the number of kept positions, or -1 on invalid parameters.
 */
int32_t orc_slice(const orc_slice_params* p, int32_t dtype, const void* keys, const void* queries,
                  orc_slice_out* out);

/* Whole-step parameters, mirroring the HIP library's parameter block. */
typedef struct {
  int32_t num_layers, batch, num_kv_heads, group, head_dim;
  int32_t capacity; /* slots per [sequence][head] row block */
  int32_t budget, buffer, obs_window, beta;
  double lambda, tau;
} orc_step_params;

/*
 * One eviction step over a batch of per-layer caches in host memory.
 * k_layers[l], v_layers[l]: [batch][kv_head][capacity][D] (dtype as above);
 * queries: [layer][batch][kv_head*G][alpha][D]; seq_start[b]: first valid slot
 * of sequence b (in/out); *n_slots: slot count of every sequence (in/out).
 * Below the trigger (*n_slots < budget + buffer) nothing changes and 0 is
 * returned. Otherwise each slice keeps min(N_b, B) tokens, written in their
 * original order to slots [B - kept, B); keep_out (nullable,
 * [layer][batch][kv_head][B]) receives source slots, -1 for padding.
 * Returns 1 when an eviction happened, -1 on invalid parameters.
 */
int32_t orc_evict_step(const orc_step_params* p, int32_t dtype, void* const* k_layers, void* const* v_layers,
                       const void* queries, int32_t* seq_start, int32_t* n_slots, int32_t* keep_out);

/* dst row j <- src row keep[j] for keep[j] >= 0 (out of place). */
void orc_gather_rows(const void* src, const int32_t* keep, int32_t n_keep, int32_t row_bytes, void* dst);

/*
 * Hole-filling compaction of one slice (the order-free layout), in place.
 * The slice's tokens are virtual slots in age order; virtual slot v < budget
 * is physical row order[v], v >= budget physical row v. keep: budget entries
 * (virtual slots, ascending, -1 before the kept ones), as the selection
 * writes them. Kept tokens below the budget stay; the kept tokens at or past
 * the budget (the movers, ascending) are copied into the physical rows below
 * the budget that no kept token occupies (the free rows, ascending); the
 * free rows left over go, ascending, to the virtual slots before the new
 * start. k_rows, v_rows: the slice's n_slots physical rows of row_bytes each.
 * Returns the new start (number of -1 entries) or -1 if order is not a
 * permutation of [0, budget) or keep is malformed.
 */
int32_t orc_holefill_slice(void* k_rows, void* v_rows, int32_t row_bytes, int32_t budget, int32_t n_slots,
                           const int32_t* keep, int32_t* order);

/* orc_slice with a per-token penalty (N entries, may be NULL) subtracted
 * from Z of the candidates: SkipKV's sentence-level deduction. */
int32_t orc_slice_penalized(const orc_slice_params* p, int32_t dtype, const void* keys, const void* queries,
                            const double* token_penalty, orc_slice_out* out);

/* Decode attention of one slice with n keys (the newest token's own
 * included): out[g][d] = sum_j w[g][j] v[j][d], w[g] = softmax over j of
 * q[g].k[j] / sqrt(head_dim). keys, values [n][head_dim], queries
 * [group][head_dim] in dtype; out [group][head_dim] and weights [group][n]
 * (nullable) in double. n == 0 gives out = 0. Returns 0, -1 on bad arguments. */
int32_t orc_decode_attention(int32_t n, int32_t head_dim, int32_t group, int32_t dtype, const void* keys,
                             const void* values, const void* queries, double* out, double* weights);

/* Sentence redundancy (SkipKV): vectors [n_sent][dim] in generation order;
 * penalty[i] = the largest cosine of sentence i with a later sentence when
 * it exceeds tau_s, else 0 (a zero vector has cosine 0 with everything). */
void orc_sentence_penalty(int32_t n_sent, int32_t dim, const float* vectors, double tau_s, double* penalty);

/*
 * Sampled selection of one slice with n valid tokens (positions 0..n-1):
 * ForesightKV's Top-K followed by multinomial sampling on caller scores. The
 * newest keep_newest tokens are kept; among the others the K = min(max(top_k,
 * budget - keep_newest), candidates) best by score (equal scores: the later
 * position) survive, and budget - keep_newest of the survivors are drawn
 * without replacement with probabilities proportional to
 * exp(score / temperature): the largest score / temperature - log(-log u)
 * (the Gumbel-top-k form of that draw; u in (0, 1) per token, equal keys:
 * the later position). With n <= budget all are kept. keep_out receives the
 * kept positions ascending; returns their count, or -1 on invalid input.
 */
int32_t orc_select_sampled(int32_t n, int32_t budget, int32_t keep_newest, int32_t top_k, double temperature,
                           const float* scores, const float* uniforms, int32_t* keep_out);

#ifdef __cplusplus
}
#endif
#endif
