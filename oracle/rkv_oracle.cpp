/*
 * CPU oracle of the R-KV decode-time eviction step — TEST INFRASTRUCTURE.
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Plain loops, double precision, single thread, host libm. Stored bf16 and
 * fp32 values widen to double exactly, so every quantity below is the
 * definition evaluated at (nearly) exact precision. It shares no code with the
 * HIP library.
 *
 * [RKV] = R-KV notes page (yoonschallenge.tistory.com/1236).
 */
#include "rkv_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

namespace {

double load(const void* base, int32_t dtype, int64_t idx) {
  if (dtype == ORC_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    std::memcpy(&f, &bits, 4);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

bool valid_slice_params(const orc_slice_params* p, int32_t dtype) {
  if (!p) return false;
  if (dtype != ORC_BF16 && dtype != ORC_F32) return false;
  if (p->n < 0 || p->head_dim <= 0 || p->group <= 0 || p->obs_window <= 0) return false;
  if (p->budget <= p->obs_window || p->beta < 0) return false;
  if (!(p->lambda >= 0.0 && p->lambda <= 1.0)) return false;
  return true;
}

}  // namespace

namespace {

int32_t slice_impl(const orc_slice_params* p, int32_t dtype, const void* keys, const void* queries,
                   const double* token_penalty, orc_slice_out* out) {
  if (!valid_slice_params(p, dtype) || !out) return -1;
  const int N = p->n, D = p->head_dim, G = p->group, A = p->obs_window, B = p->budget;

  /* [RKV] opening notes and summary table row "decoding-time compression":
   * a slice that has not outgrown the budget keeps every token. */
  if (N <= B) {
    if (out->keep)
      for (int j = 0; j < N; ++j) out->keep[j] = j;
    return N;
  }
  if (!keys || !queries) return -1;

  /* Partition: the newest A tokens are the observation window O = [N-A, N),
   * kept unconditionally; the rest are the candidates C = [0, N-A). */
  const int nc = N - A;

  std::vector<double> K((size_t)N * D);
  for (int64_t i = 0; i < (int64_t)N * D; ++i) K[i] = load(keys, dtype, i);

  /* Importance ([RKV] notes; summary table row "importance computation"):
   * the attention weight that each observation query puts on key j, i.e. a
   * causal softmax over keys 0..p of q.k/sqrt(D) for the query at position
   * p = N-A+t; averaged over the A observation queries of one query head,
   * then max-pooled over the G query heads sharing the KV head. */
  std::vector<double> imp(N, 0.0), ibar(N), logit(N);
  const double inv_sqrt_d = 1.0 / std::sqrt((double)D);
  for (int g = 0; g < G; ++g) {
    std::fill(ibar.begin(), ibar.end(), 0.0);
    for (int t = 0; t < A; ++t) {
      const int pos = N - A + t;
      std::vector<double> q(D);
      for (int d = 0; d < D; ++d) q[d] = load(queries, dtype, (int64_t)(g * A + t) * D + d);
      double mx = -INFINITY;
      for (int j = 0; j <= pos; ++j) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += q[d] * K[(size_t)j * D + d];
        logit[j] = s * inv_sqrt_d;
        mx = std::max(mx, logit[j]);
      }
      double den = 0.0;
      for (int j = 0; j <= pos; ++j) den += std::exp(logit[j] - mx);
      for (int j = 0; j <= pos; ++j) ibar[j] += (std::exp(logit[j] - mx) / den) / A;
    }
    for (int j = 0; j < N; ++j) imp[j] = (g == 0) ? ibar[j] : std::max(imp[j], ibar[j]);
  }

  /* Key normalisation ([RKV] Q&A cause 3, the list of per-128-token work):
   * khat_j = k_j / ||k_j||, and khat_j = 0 for a zero key. */
  std::vector<double> Kh((size_t)N * D, 0.0);
  for (int j = 0; j < N; ++j) {
    double ss = 0.0;
    for (int d = 0; d < D; ++d) ss += K[(size_t)j * D + d] * K[(size_t)j * D + d];
    double nrm = std::sqrt(ss);
    if (nrm > 0.0)
      for (int d = 0; d < D; ++d) Kh[(size_t)j * D + d] = K[(size_t)j * D + d] / nrm;
  }

  /* Redundancy ([RKV] notes; summary table row "redundancy computation"):
   * S_ij = khat_i . khat_j over every valid pair i != j of the slice. A token
   * similar to many others is redundant; among similar tokens the beta most
   * recent are protected. Reading: "similar" is S_ij > tau; token i is
   * protected iff fewer than beta tokens newer than i are similar to it, and
   * a protected token gets redundancy 0. The unprotected redundancy is the
   * mean similarity to the other N-1 tokens. S_ji is S_ij (the same products
   * summed in the same order), so each pair is evaluated once. */
  std::vector<double> rowsum(N, 0.0);
  std::vector<int32_t> cnt(N, 0), amb(N, 0);
  for (int i = 0; i < N; ++i) {
    for (int j = i + 1; j < N; ++j) {
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += Kh[(size_t)i * D + d] * Kh[(size_t)j * D + d];
      rowsum[i] += s;
      rowsum[j] += s;
      if (s > p->tau) cnt[i] += 1;
      if (std::fabs(s - p->tau) <= p->amb_eps) amb[i] = 1;
    }
  }
  std::vector<double> rowmean(N), rbar(N);
  for (int i = 0; i < N; ++i) {
    rowmean[i] = rowsum[i] / (double)(N - 1);
    rbar[i] = (cnt[i] < p->beta) ? 0.0 : rowmean[i];
  }

  /* [RKV] Q&A cause 3: a softmax over the redundancy scores (of the
   * candidates), then the combination. The combination formula did not
   * survive on the page (summary table row "final selection criterion" keeps
   * only: importance raises the score, redundancy lowers it, lambda = 0.1 was
   * best). Reading: Z = lambda*I - (1-lambda)*R. */
  std::vector<double> R(N, 0.0), Z(N, 0.0);
  double rmax = -INFINITY;
  for (int i = 0; i < nc; ++i) rmax = std::max(rmax, rbar[i]);
  double rden = 0.0;
  for (int i = 0; i < nc; ++i) rden += std::exp(rbar[i] - rmax);
  for (int i = 0; i < nc; ++i) {
    R[i] = std::exp(rbar[i] - rmax) / rden;
    Z[i] = p->lambda * imp[i] - (1.0 - p->lambda) * R[i];
    /* [SKV] SkipKV notes page, summary table row "final eviction score":
     * tokens of redundant sentences lose their sentence's similarity on top. */
    if (token_penalty) Z[i] -= token_penalty[i];
  }

  /* Selection ([RKV] opening notes: keep the newest 8, score the rest, keep
   * the top tokens that fit the budget). Reading: the budget includes the
   * observation window, so k = B - A candidates are chosen by Z descending;
   * equal Z goes to the more recent position. Output in ascending order. */
  const int k = B - A;
  std::vector<int32_t> order(nc);
  for (int i = 0; i < nc; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (Z[a] != Z[b]) return Z[a] > Z[b];
    return a > b;
  });
  std::vector<int32_t> kept(order.begin(), order.begin() + k);
  for (int j = nc; j < N; ++j) kept.push_back(j);
  std::sort(kept.begin(), kept.end());

  for (int i = 0; i < N; ++i) {
    if (out->importance) out->importance[i] = imp[i];
    if (out->rowmean) out->rowmean[i] = rowmean[i];
    if (out->counts) out->counts[i] = cnt[i];
    if (out->rbar) out->rbar[i] = rbar[i];
    if (out->R) out->R[i] = R[i];
    if (out->Z) out->Z[i] = Z[i];
    if (out->ambiguous) out->ambiguous[i] = amb[i];
  }
  if (out->keep)
    for (int j = 0; j < B; ++j) out->keep[j] = kept[j];
  return B;
}

}  // namespace

extern "C" int32_t orc_slice(const orc_slice_params* p, int32_t dtype, const void* keys, const void* queries,
                             orc_slice_out* out) {
  return slice_impl(p, dtype, keys, queries, nullptr, out);
}

extern "C" int32_t orc_slice_penalized(const orc_slice_params* p, int32_t dtype, const void* keys,
                                       const void* queries, const double* token_penalty, orc_slice_out* out) {
  return slice_impl(p, dtype, keys, queries, token_penalty, out);
}

/* Decode attention of one slice, the step that runs at every generated token
 * ([RKV] Q&A part 2, cause 4: fusing attention, importance scoring and
 * eviction into one kernel). The newest token's G query heads attend to the
 * slice's n keys, its own key included: w_gj = softmax over j of
 * q_g.k_j / sqrt(D), and out_g = sum_j w_gj v_j. The weights are the
 * attention rows that the importance averages over the observation window,
 * so a decode step can hand them over as it computes them. */
extern "C" int32_t orc_decode_attention(int32_t n, int32_t head_dim, int32_t group, int32_t dtype, const void* keys,
                                        const void* values, const void* queries, double* out, double* weights) {
  if (n < 0 || head_dim <= 0 || group <= 0 || !out) return -1;
  if (dtype != ORC_BF16 && dtype != ORC_F32) return -1;
  const int D = head_dim;
  for (int64_t i = 0; i < (int64_t)group * D; ++i) out[i] = 0.0;
  if (n == 0) return 0;
  if (!keys || !values || !queries) return -1;
  const double inv_sqrt_d = 1.0 / std::sqrt((double)D);
  std::vector<double> lg(n);
  for (int g = 0; g < group; ++g) {
    double mx = -INFINITY;
    for (int j = 0; j < n; ++j) {
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += load(queries, dtype, (int64_t)g * D + d) * load(keys, dtype, (int64_t)j * D + d);
      lg[j] = inv_sqrt_d * s;
      mx = std::max(mx, lg[j]);
    }
    double den = 0.0;
    for (int j = 0; j < n; ++j) den += std::exp(lg[j] - mx);
    for (int j = 0; j < n; ++j) {
      const double w = std::exp(lg[j] - mx) / den;
      if (weights) weights[(int64_t)g * n + j] = w;
      for (int d = 0; d < D; ++d) out[(int64_t)g * D + d] += w * load(values, dtype, (int64_t)j * D + d);
    }
  }
  return 0;
}

extern "C" void orc_sentence_penalty(int32_t n_sent, int32_t dim, const float* vectors, double tau_s,
                                     double* penalty) {
  /* [SKV] SkipKV notes page, summary table row "sentence-level KV storage
   * skipping": a sentence is represented by the mean of its tokens' last-layer
   * hidden states (the vectors given here); when a later sentence's cosine
   * with an earlier one exceeds the threshold, the earlier one is redundant.
   * Reading: its penalty is the largest such cosine, 0 if none exceeds. */
  std::vector<double> nrm(n_sent, 0.0);
  for (int i = 0; i < n_sent; ++i) {
    double ss = 0.0;
    for (int d = 0; d < dim; ++d) ss += (double)vectors[(size_t)i * dim + d] * vectors[(size_t)i * dim + d];
    nrm[i] = std::sqrt(ss);
  }
  for (int i = 0; i < n_sent; ++i) {
    double best = 0.0;
    bool any = false;
    for (int j = i + 1; j < n_sent; ++j) {
      if (nrm[i] == 0.0 || nrm[j] == 0.0) continue;
      double dot = 0.0;
      for (int d = 0; d < dim; ++d) dot += (double)vectors[(size_t)i * dim + d] * vectors[(size_t)j * dim + d];
      const double c = dot / (nrm[i] * nrm[j]);
      if (c > tau_s && (!any || c > best)) {
        best = c;
        any = true;
      }
    }
    penalty[i] = any ? best : 0.0;
  }
}

extern "C" void orc_gather_rows(const void* src, const int32_t* keep, int32_t n_keep, int32_t row_bytes,
                                void* dst) {
  /* [RKV] Q&A cause 3: the selected KV is copied into the new cache. */
  for (int32_t j = 0; j < n_keep; ++j)
    if (keep[j] >= 0)
      std::memcpy((char*)dst + (size_t)j * row_bytes, (const char*)src + (size_t)keep[j] * row_bytes,
                  (size_t)row_bytes);
}

extern "C" int32_t orc_evict_step(const orc_step_params* p, int32_t dtype, void* const* k_layers,
                                  void* const* v_layers, const void* queries, int32_t* seq_start, int32_t* n_slots,
                                  int32_t* keep_out) {
  if (!p || !k_layers || !v_layers || !queries || !seq_start || !n_slots) return -1;
  if (dtype != ORC_BF16 && dtype != ORC_F32) return -1;
  const int L = p->num_layers, Bt = p->batch, H = p->num_kv_heads, G = p->group, D = p->head_dim;
  const int C = p->capacity, B = p->budget, A = p->obs_window;
  if (L <= 0 || Bt <= 0 || H <= 0 || G <= 0 || D <= 0) return -1;
  if (B <= A || p->buffer <= 0 || B + p->buffer > C || *n_slots > C || *n_slots < 0) return -1;
  for (int b = 0; b < Bt; ++b)
    if (seq_start[b] < 0 || seq_start[b] > *n_slots) return -1;

  /* [RKV] summary table row "decoding-time compression": compression runs
   * when budget + buffer slots are full (buffer 128 by default). Reading for
   * a batch: the shared slot count triggers it; below it nothing changes. */
  if (*n_slots < B + p->buffer) return 0;

  const int esz = dtype == ORC_BF16 ? 2 : 4;
  const int row_bytes = D * esz;
  orc_slice_params sp;
  sp.head_dim = D;
  sp.group = G;
  sp.obs_window = A;
  sp.budget = B;
  sp.beta = p->beta;
  sp.lambda = p->lambda;
  sp.tau = p->tau;
  sp.amb_eps = 0.0;
  std::vector<int32_t> keep(B);
  std::vector<char> orig;
  for (int l = 0; l < L; ++l)
    for (int b = 0; b < Bt; ++b)
      for (int h = 0; h < H; ++h) {
        const int s0 = seq_start[b];
        const int N = *n_slots - s0;
        const size_t slice_off = ((size_t)b * H + h) * (size_t)C * row_bytes;
        char* kbase = (char*)k_layers[l] + slice_off;
        char* vbase = (char*)v_layers[l] + slice_off;
        const char* qblk = (const char*)queries + ((((size_t)l * Bt + b) * H + h) * (size_t)G * A) * row_bytes;
        sp.n = N;
        orc_slice_out so;
        std::memset(&so, 0, sizeof(so));
        so.keep = keep.data();
        const int kept = orc_slice(&sp, dtype, kbase + (size_t)s0 * row_bytes, qblk, &so);
        if (kept < 0) return -1;
        /* source slots, padded on the left with -1, destination [B-kept, B) */
        std::vector<int32_t> src(B, -1);
        for (int j = 0; j < kept; ++j) src[B - kept + j] = s0 + keep[j];
        if (keep_out) std::memcpy(keep_out + (((size_t)l * Bt + b) * H + h) * B, src.data(), sizeof(int32_t) * B);
        char* bases[2] = {kbase, vbase};
        for (char* base : bases) {
          orig.assign(base, base + (size_t)(*n_slots) * row_bytes);
          orc_gather_rows(orig.data(), src.data(), B, row_bytes, base);
        }
      }
  for (int b = 0; b < Bt; ++b) {
    const int N = *n_slots - seq_start[b];
    seq_start[b] = B - std::min(N, B);
  }
  *n_slots = B;
  return 1;
}

extern "C" int32_t orc_holefill_slice(void* k_rows, void* v_rows, int32_t row_bytes, int32_t budget,
                                      int32_t n_slots, const int32_t* keep, int32_t* order) {
  /* [RKV] Q&A part 2, causes 3 and 4: copying the selected KV and
   * re-arranging the cache are the costs after pruning; this layout copies
   * only the kept tokens that arrived after the budget. Which free row a
   * mover takes is a stated choice (ascending to ascending). */
  const int B = budget;
  std::vector<int> seen(B, 0);
  for (int v = 0; v < B; ++v) {
    if (order[v] < 0 || order[v] >= B || seen[order[v]]) return -1;
    seen[order[v]] = 1;
  }
  int lead = 0;
  while (lead < B && keep[lead] < 0) ++lead;
  for (int j = lead; j < B; ++j)
    if (keep[j] < 0 || keep[j] >= n_slots || (j > lead && keep[j] <= keep[j - 1])) return -1;
  // rows occupied by the kept tokens that stay
  std::vector<int> occupied(B, 0);
  for (int j = lead; j < B; ++j)
    if (keep[j] < B) occupied[order[keep[j]]] = 1;
  std::vector<int> free_rows;
  for (int r = 0; r < B; ++r)
    if (!occupied[r]) free_rows.push_back(r);
  std::vector<int> new_order(B, -1);
  int m = 0;  // movers so far
  for (int j = lead; j < B; ++j) {
    if (keep[j] < B) {
      new_order[j] = order[keep[j]];
    } else {
      const int dst = free_rows[m++];
      std::memcpy((char*)k_rows + (size_t)dst * row_bytes, (const char*)k_rows + (size_t)keep[j] * row_bytes,
                  (size_t)row_bytes);
      std::memcpy((char*)v_rows + (size_t)dst * row_bytes, (const char*)v_rows + (size_t)keep[j] * row_bytes,
                  (size_t)row_bytes);
      new_order[j] = dst;
    }
  }
  for (int j = 0; j < lead; ++j) new_order[j] = free_rows[m + j];
  for (int v = 0; v < B; ++v) order[v] = new_order[v];
  return lead;
}

extern "C" int32_t orc_select_sampled(int32_t n, int32_t budget, int32_t keep_newest, int32_t top_k,
                                      double temperature, const float* scores, const float* uniforms,
                                      int32_t* keep_out) {
  /* [FKV] ForesightKV explainer, technical summary: keep the newest L
   * tokens, compress the rest to B - L; Top-K, then multinomial sampling. */
  if (n < 0 || budget < 1 || keep_newest < 0 || keep_newest >= budget || top_k < 0 || !(temperature > 0.0))
    return -1;
  if (n <= budget) {
    for (int j = 0; j < n; ++j) keep_out[j] = j;
    return n;
  }
  const int nc = n - keep_newest, kk = budget - keep_newest;
  const int K = std::min(std::max(top_k, kk), nc);
  // the top K candidates by score, equal scores to the later position
  std::vector<int> cand(nc);
  for (int i = 0; i < nc; ++i) cand[i] = i;
  std::sort(cand.begin(), cand.end(), [&](int a, int b) {
    const double sa = scores[a], sb = scores[b];
    return sa != sb ? sa > sb : a > b;
  });
  cand.resize(K);
  // a draw of kk without replacement, probabilities proportional to
  // exp(score / T): the kk largest Gumbel-perturbed keys
  std::vector<double> key(nc, 0.0);
  for (int i : cand) key[i] = (double)scores[i] / temperature - std::log(-std::log((double)uniforms[i]));
  std::sort(cand.begin(), cand.end(), [&](int a, int b) { return key[a] != key[b] ? key[a] > key[b] : a > b; });
  std::vector<int> kept(cand.begin(), cand.begin() + kk);
  for (int j = nc; j < n; ++j) kept.push_back(j);
  std::sort(kept.begin(), kept.end());
  for (int j = 0; j < budget; ++j) keep_out[j] = kept[j];
  return budget;
}
