/*
 * ts_oracle.c -- fp64 CPU oracle for causal grouped-query prefill attention
 * with an optional sliding window and a per-head attention sink.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library.  It shares no
 * source, header, table or helper with the HIP implementation, and it must
 * never be used as a fallback for it.
 *
 * What is computed (sources, cited by page and section):
 *  - "TokenSpeed-kernel multi-silicon" (aixai.ru blog), section
 *    "Числа: Gluon на AMD MI355X": the GPT-OSS attention being served is
 *    regular multi-head attention with attention sinks and a mix of
 *    sliding-window and full-attention layers; the prefill case measured there
 *    is full causal with bf16 Q/K/V, head_dim 64, 64 query heads over 8 KV
 *    heads (so each KV head serves a group of query heads).
 *  - ai-radar.it article on TokenSpeed-kernel, section
 *    "AMD MI355X: la prova sul campo": attention with a sliding window and
 *    attention sinks.
 *  - TokenSpeed-kernel README, section "Public API": `mha_prefill` is listed
 *    apart from `mha_prefill_with_kvcache`, so this operation attends only
 *    within the packed sequences it is given (no cache).
 *
 * The pages print no formula.  The readings taken here (all listed with their
 * reasons in the design notes):
 *  - sink: one fp32 logit per query head, in the same (already scaled) units
 *    as the scores and with the natural exponential; it joins the softmax
 *    denominator and contributes no value row.  NULL means no sink.
 *  - window W > 0: key j is visible to query i iff 0 <= i - j < W (the query
 *    itself plus W-1 earlier keys); W <= 0 means plain causal.
 *  - positions are relative to each packed sequence; query and key share
 *    them, so the causal diagonal is j <= i.
 *  - query head h reads KV head floor(h / G), G = n_q_heads / n_kv_heads.
 *  - layout: packed rows, q/out [T][n_q_heads][D], k/v [T][n_kv_heads][D],
 *    sequence b spans rows cu_seqlens[b] .. cu_seqlens[b+1]-1.
 *
 * For row (b, i, h), with s = cu_seqlens[b] and A_i the visible keys:
 *     z_j   = scale * sum_d q[s+i][h][d] * k[s+j][g][d]          (j in A_i)
 *     m     = max(sigma_h, max_j z_j)
 *     den   = exp(sigma_h - m) + sum_j exp(z_j - m)
 *     out_d = sum_j exp(z_j - m) * v[s+j][g][d] / den
 * i.e. the plain softmax definition written out: two passes per row (scores
 * and their maximum, then exponentials, sums and the weighted average of V),
 * every operation in double precision on bf16 inputs widened exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TS_ORACLE_OK 0
#define TS_ORACLE_BAD_ARGS (-1)
#define TS_ORACLE_NO_MEMORY (-2)

/* bf16 bit pattern -> double.  A bf16 number is the upper half of an IEEE
 * binary32 number, so widening is exact. */
static double bf16_to_double(uint16_t bits) {
  uint32_t w = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static int check_args(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* cu_seqlens, int32_t n_seqs,
                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      double scale) {
  if (!cu_seqlens || n_seqs < 0) return TS_ORACLE_BAD_ARGS;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0) return TS_ORACLE_BAD_ARGS;
  if (n_q_heads % n_kv_heads != 0) return TS_ORACLE_BAD_ARGS;
  if (!(scale > 0.0) || !isfinite(scale)) return TS_ORACLE_BAD_ARGS;
  if (cu_seqlens[0] != 0) return TS_ORACLE_BAD_ARGS;
  for (int32_t b = 0; b < n_seqs; ++b)
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return TS_ORACLE_BAD_ARGS;
  if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v)) return TS_ORACLE_BAD_ARGS;
  return TS_ORACLE_OK;
}

/* Sequence that holds packed row t (cu_seqlens is non-decreasing). */
static int32_t seq_of_row(const int32_t* cu_seqlens, int32_t n_seqs, int64_t t) {
  int32_t lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) / 2;
    if (cu_seqlens[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* First visible key position for query position i. */
static int64_t first_visible(int64_t i, int32_t window) {
  if (window <= 0) return 0;
  int64_t lo = i - (int64_t)window + 1;
  return lo > 0 ? lo : 0;
}

/* One output row.  z is caller scratch of at least (i+1) doubles, acc of
 * head_dim doubles.  Also returns the probabilities when probs != NULL
 * (probs[j] for j in A_i, zero elsewhere in [0, i]) and the sink's share. */
static void one_row(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const float* sinks, int64_t s, int64_t i, int32_t h,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    int32_t window, double scale, double* z, double* acc,
                    double* out_row, double* probs, double* p_sink) {
  const int32_t G = n_q_heads / n_kv_heads;
  const int32_t g = h / G;
  const int64_t jlo = first_visible(i, window);
  const double sigma = sinks ? (double)sinks[h] : -INFINITY;
  const uint16_t* qrow = q + ((s + i) * n_q_heads + h) * (int64_t)head_dim;

  /* pass 1: scaled scores and the maximum, sink included */
  double m = sigma;
  for (int64_t j = jlo; j <= i; ++j) {
    const uint16_t* krow = k + ((s + j) * n_kv_heads + g) * (int64_t)head_dim;
    double dot = 0.0;
    for (int32_t d = 0; d < head_dim; ++d)
      dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
    z[j - jlo] = scale * dot;
    if (z[j - jlo] > m) m = z[j - jlo];
  }

  /* pass 2: exponentials, denominator, weighted sum of V rows */
  double den = (sigma == -INFINITY) ? 0.0 : exp(sigma - m);
  for (int32_t d = 0; d < head_dim; ++d) acc[d] = 0.0;
  for (int64_t j = jlo; j <= i; ++j) {
    const double w = exp(z[j - jlo] - m);
    const uint16_t* vrow = v + ((s + j) * n_kv_heads + g) * (int64_t)head_dim;
    den += w;
    for (int32_t d = 0; d < head_dim; ++d) acc[d] += w * bf16_to_double(vrow[d]);
    z[j - jlo] = w;
  }
  if (out_row)
    for (int32_t d = 0; d < head_dim; ++d) out_row[d] = acc[d] / den;
  if (probs) {
    for (int64_t j = 0; j <= i; ++j) probs[j] = 0.0;
    for (int64_t j = jlo; j <= i; ++j) probs[j] = z[j - jlo] / den;
  }
  if (p_sink) *p_sink = (sigma == -INFINITY) ? 0.0 : exp(sigma - m) / den;
}

/* Full output, out[T][n_q_heads][head_dim] in double. */
int ts_oracle_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const float* sinks, const int32_t* cu_seqlens,
                      int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                      int32_t head_dim, int32_t window, double scale,
                      double* out) {
  int rc = check_args(q, k, v, cu_seqlens, n_seqs, n_q_heads, n_kv_heads, head_dim, scale);
  if (rc) return rc;
  const int64_t T = cu_seqlens[n_seqs];
  if (T == 0) return TS_ORACLE_OK;
  if (!out) return TS_ORACLE_BAD_ARGS;
  int64_t max_len = 0;
  for (int32_t b = 0; b < n_seqs; ++b)
    if (cu_seqlens[b + 1] - cu_seqlens[b] > max_len) max_len = cu_seqlens[b + 1] - cu_seqlens[b];
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)max_len);
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!z || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < T * n_q_heads; ++r) {
        const int64_t t = r / n_q_heads;
        const int32_t h = (int32_t)(r % n_q_heads);
        const int32_t b = seq_of_row(cu_seqlens, n_seqs, t);
        const int64_t s = cu_seqlens[b];
        one_row(q, k, v, sinks, s, t - s, h, n_q_heads, n_kv_heads, head_dim, window,
                scale, z, acc, out + r * (int64_t)head_dim, NULL, NULL);
      }
    }
    free(z);
    free(acc);
  }
  return failed ? TS_ORACLE_NO_MEMORY : TS_ORACLE_OK;
}

/* Selected rows only: row n is (packed row rows[n], query head heads[n]);
 * out[n][head_dim].  Used where the full output is too costly on a CPU. */
int ts_oracle_prefill_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* sinks, const int32_t* cu_seqlens,
                           int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, int32_t window, double scale,
                           const int64_t* rows, const int32_t* heads, int64_t n_rows,
                           double* out) {
  int rc = check_args(q, k, v, cu_seqlens, n_seqs, n_q_heads, n_kv_heads, head_dim, scale);
  if (rc) return rc;
  if (n_rows < 0 || (n_rows > 0 && (!rows || !heads || !out))) return TS_ORACLE_BAD_ARGS;
  const int64_t T = cu_seqlens[n_seqs];
  for (int64_t n = 0; n < n_rows; ++n)
    if (rows[n] < 0 || rows[n] >= T || heads[n] < 0 || heads[n] >= n_q_heads) return TS_ORACLE_BAD_ARGS;
  int64_t max_len = 0;
  for (int32_t b = 0; b < n_seqs; ++b)
    if (cu_seqlens[b + 1] - cu_seqlens[b] > max_len) max_len = cu_seqlens[b + 1] - cu_seqlens[b];
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!z || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t n = 0; n < n_rows; ++n) {
        const int32_t b = seq_of_row(cu_seqlens, n_seqs, rows[n]);
        const int64_t s = cu_seqlens[b];
        one_row(q, k, v, sinks, s, rows[n] - s, heads[n], n_q_heads, n_kv_heads, head_dim,
                window, scale, z, acc, out + n * (int64_t)head_dim, NULL, NULL);
      }
    }
    free(z);
    free(acc);
  }
  return failed ? TS_ORACLE_NO_MEMORY : TS_ORACLE_OK;
}

/* Softmax weights of one row: probs[j] for key positions j = 0..i of the row's
 * sequence (zero where invisible) and the sink's share in *p_sink.  These are
 * the weights that the output row averages V with. */
int ts_oracle_row_probs(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* sinks, const int32_t* cu_seqlens,
                        int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, int32_t window, double scale,
                        int64_t row, int32_t head, double* probs, double* p_sink) {
  int rc = check_args(q, k, v, cu_seqlens, n_seqs, n_q_heads, n_kv_heads, head_dim, scale);
  if (rc) return rc;
  const int64_t T = cu_seqlens[n_seqs];
  if (row < 0 || row >= T || head < 0 || head >= n_q_heads || !probs || !p_sink) return TS_ORACLE_BAD_ARGS;
  const int32_t b = seq_of_row(cu_seqlens, n_seqs, row);
  const int64_t s = cu_seqlens[b];
  const int64_t i = row - s;
  double* z = (double*)malloc(sizeof(double) * (size_t)(i + 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
  if (!z || !acc) { free(z); free(acc); return TS_ORACLE_NO_MEMORY; }
  one_row(q, k, v, sinks, s, i, head, n_q_heads, n_kv_heads, head_dim, window, scale,
          z, acc, NULL, probs, p_sink);
  free(z);
  free(acc);
  return TS_ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Attention of new query rows against a paged KV cache.
 *
 * Pages followed: TokenSpeed-kernel README, section "Public API", which lists
 * `mha_prefill_with_kvcache` and `mha_decode_with_kvcache` beside
 * `mha_prefill`; "TokenSpeed-kernel multi-silicon" (aixai.ru blog), section
 * "Архитектура: три слоя", where the runtime's attention calls are prefill and
 * decode with a KV cache.  The pages print no signature; the readings taken:
 *  - the cache holds every key and value of a sequence, the new tokens' own
 *    included (the caller writes them before the call); seqlens_k[b] counts
 *    them all;
 *  - layout: k_cache / v_cache [n_pages][page_size][n_kv_heads][D]; key
 *    position j of sequence b lives in page block_table[b][j / page_size],
 *    slot j % page_size;
 *  - the q_len = cu_seqlens_q[b+1] - cu_seqlens_q[b] new query rows are the
 *    last q_len positions of the sequence: row i sits at position
 *    p = seqlens_k[b] - q_len + i (the causal diagonal aligned to the bottom
 *    right); decode is q_len = 1;
 *  - visible keys, sink, scale and GQA mapping as in the prefill above, with
 *    p in place of i; a row with p < 0 (fewer cached keys than new rows) sees
 *    no key and its output is zero.
 * ------------------------------------------------------------------------ */

/* One output row of the cache form; z holds at least p+1 doubles. */
static int cache_row(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                     const float* sinks, const int32_t* block_table, int32_t b, int64_t p,
                     int64_t t, int32_t h, int32_t n_pages, int32_t page_size,
                     int32_t pages_per_seq, int32_t n_q_heads, int32_t n_kv_heads,
                     int32_t head_dim, int32_t window, double scale, double* z, double* acc,
                     double* out_row) {
  const int32_t G = n_q_heads / n_kv_heads;
  const int32_t g = h / G;
  for (int32_t d = 0; d < head_dim; ++d) out_row[d] = 0.0;
  if (p < 0) return TS_ORACLE_OK;
  const int64_t jlo = first_visible(p, window);
  const double sigma = sinks ? (double)sinks[h] : -INFINITY;
  const uint16_t* qrow = q + (t * n_q_heads + h) * (int64_t)head_dim;
  const int32_t* pages = block_table + (int64_t)b * pages_per_seq;

  /* pass 1: scaled scores and the maximum, sink included */
  double m = sigma;
  for (int64_t j = jlo; j <= p; ++j) {
    const int64_t slot = j % page_size;
    const int64_t pi = j / page_size;
    if (pi >= pages_per_seq || pages[pi] < 0 || pages[pi] >= n_pages) return TS_ORACLE_BAD_ARGS;
    const uint16_t* krow = k_cache + (((int64_t)pages[pi] * page_size + slot) * n_kv_heads + g) * head_dim;
    double dot = 0.0;
    for (int32_t d = 0; d < head_dim; ++d)
      dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
    z[j - jlo] = scale * dot;
    if (z[j - jlo] > m) m = z[j - jlo];
  }

  /* pass 2: exponentials, denominator (sink term first), weighted sum of V rows */
  double den = sinks ? exp(sigma - m) : 0.0;
  for (int32_t d = 0; d < head_dim; ++d) acc[d] = 0.0;
  for (int64_t j = jlo; j <= p; ++j) {
    const double w = exp(z[j - jlo] - m);
    const uint16_t* vrow = v_cache + (((int64_t)pages[j / page_size] * page_size + j % page_size) * n_kv_heads + g) * head_dim;
    den += w;
    for (int32_t d = 0; d < head_dim; ++d) acc[d] += w * bf16_to_double(vrow[d]);
  }
  for (int32_t d = 0; d < head_dim; ++d) out_row[d] = acc[d] / den;
  return TS_ORACLE_OK;
}

/* Rows of the cache form.  q and out are packed [Tq][n_q_heads][D] by
 * cu_seqlens_q (Tq = cu_seqlens_q[n_seqs]).  With rows == NULL every
 * (row, head) is computed into out[Tq][n_q_heads][D]; otherwise row n is
 * (packed row rows[n], head heads[n]) into out[n][D]. */
int ts_oracle_cache(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    const float* sinks, const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                    const int32_t* block_table, int32_t n_seqs, int32_t n_pages,
                    int32_t page_size, int32_t pages_per_seq, int32_t n_q_heads,
                    int32_t n_kv_heads, int32_t head_dim, int32_t window, double scale,
                    const int64_t* rows, const int32_t* heads, int64_t n_rows, double* out) {
  int rc = check_args(q, k_cache, v_cache, cu_seqlens_q, n_seqs, n_q_heads, n_kv_heads, head_dim, scale);
  if (rc) return rc;
  if (!seqlens_k || n_pages < 0 || page_size <= 0 || pages_per_seq < 0) return TS_ORACLE_BAD_ARGS;
  int64_t max_len = 1;
  for (int32_t b = 0; b < n_seqs; ++b) {
    if (seqlens_k[b] < 0 || (int64_t)seqlens_k[b] > (int64_t)pages_per_seq * page_size) return TS_ORACLE_BAD_ARGS;
    if (seqlens_k[b] > max_len) max_len = seqlens_k[b];
  }
  if (n_seqs > 0 && pages_per_seq > 0 && !block_table) return TS_ORACLE_BAD_ARGS;
  const int64_t Tq = cu_seqlens_q[n_seqs];
  const int64_t n = rows ? n_rows : Tq * n_q_heads;
  if (n < 0 || (n > 0 && !out) || (rows && n > 0 && !heads)) return TS_ORACLE_BAD_ARGS;
  if (rows)
    for (int64_t r = 0; r < n; ++r)
      if (rows[r] < 0 || rows[r] >= Tq || heads[r] < 0 || heads[r] >= n_q_heads) return TS_ORACLE_BAD_ARGS;
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)max_len);
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!z || !acc) {
#pragma omp atomic write
      failed = TS_ORACLE_NO_MEMORY;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < n; ++r) {
        const int64_t t = rows ? rows[r] : r / n_q_heads;
        const int32_t h = rows ? heads[r] : (int32_t)(r % n_q_heads);
        const int32_t b = seq_of_row(cu_seqlens_q, n_seqs, t);
        const int64_t q_len = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        const int64_t p = (int64_t)seqlens_k[b] - q_len + (t - cu_seqlens_q[b]);
        const int rr = cache_row(q, k_cache, v_cache, sinks, block_table, b, p, t, h, n_pages,
                                 page_size, pages_per_seq, n_q_heads, n_kv_heads, head_dim, window,
                                 scale, z, acc, out + r * (int64_t)head_dim);
        if (rr) {
#pragma omp atomic write
          failed = rr;
        }
      }
    }
    free(z);
    free(acc);
  }
  return failed;
}
