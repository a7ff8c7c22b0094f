/*
 * oracle/decode_ref.c -- plain, slow, float64 CPU reference for single-query
 * GQA decode attention over a contiguous or a paged K/V cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (for every request b and query/output head h):
 *   g      = h / (Hq / Hkv)                      -- consecutive query heads share a
 *                                                   KV head (ferrox-cuda 0.15.2
 *                                                   src/attn.rs, kernel source
 *                                                   gqa_decode: the group index)
 *   x_j    = scale * <q[b,h,:], K_b[g,j,:]>       j = 0 .. L_b-1
 *   o      = sum_j softmax(x)_j * V_b[g,j,:]      (ferrum-kernels 0.7.7
 *                                                   src/backend/cuda/decode_attention.rs,
 *                                                   module doc: scores, stable
 *                                                   softmax, weighted sum of V)
 *   lse    = ln sum_j exp(x_j)                    (baracuda-kernels 0.0.1-alpha.68
 *                                                   src/attention/batch_paged_decode.rs,
 *                                                   module doc "Query / output": a
 *                                                   per-row log-sum-exp kept in f32)
 * The softmax is evaluated in the textbook two-pass way: pass 1 finds the max
 * score M, pass 2 sums w_j = exp(x_j - M) and the w_j-weighted V rows.
 *
 * Readings taken where the pages are silent:
 *   - lse is the natural log of the sum of exp of the *scaled* scores.
 *   - a request with no valid rows yields o = 0 and lse = -inf (the ferrox-cuda
 *     page returns zeros for an empty sequence; log of an empty sum is -inf).
 *   - paged: request b owns pages indices[indptr[b] .. indptr[b+1]); all but the
 *     last are full, the last holds last_page_len[b] rows, so
 *     L_b = (n_b - 1) * page_size + last_page_len[b] for n_b >= 1, and 0 for n_b = 0
 *     (baracuda-kernels page, module doc "Layout").
 *   - K/V rows outside [0, L_b) are excluded, never down-weighted.
 *
 * Element decoding is exact: f32 is widened, bf16 is the high half of an f32,
 * f16 is decoded from its sign / exponent / mantissa fields by hand.
 *
 * Two variants of the scores that the baracuda-kernels page lists as not
 * supported by its plan (module doc "Constraints"), with the readings taken:
 *   window > 0:  a sliding window -- the query, the request's newest token at
 *                position L_b - 1, sees only the last `window` rows,
 *                j >= L_b - window (0: every row);
 *   softcap > 0: logits soft-capping -- each scaled score x_j becomes
 *                softcap * tanh(x_j / softcap), and lse sums exp of the capped
 *                scores (0: off);
 *   alibi:       per query head slopes m_h (NULL: off) -- the score of row j
 *                gains m_h * (j - (L_b - 1)), a linear penalty on the distance
 *                back from the query's own position, added to the scaled score
 *                before any cap;
 *   mask:        a custom mask (NULL: off), one bit per K/V row of every
 *                request, requests back to back in request order: row j of
 *                request b is bit R_b + j with R_b = L_0 + .. + L_{b-1} (for
 *                a contiguous cache, bit j), bit i at byte i / 8, bit i % 8.
 *                A set bit keeps the row, a clear bit removes it from the
 *                softmax as if it were not there (positions, and so ALiBi
 *                distances, of the kept rows do not change).  Rows must pass
 *                both the window and the mask; a query with no row left gets
 *                o = 0 and lse = -inf.  The baracuda-kernels page lists custom
 *                masks as not supported without defining one; this reading
 *                is the plainest for a single query row per request.
 *
 * Two K/V layouts (argument `layout`):
 *   OR_HND (0), heads-major: contiguous [Hkv, max_kv_len, D] (ferrum-kernels
 *     page, decode_attention argument list), paged [pages, Hkv, P, D]
 *     (baracuda-kernels page, module doc "Layout");
 *   OR_NHD (1), token-major: contiguous [max_kv_len, Hkv, D], row t of KV head g
 *     at (t * Hkv + g) * D (ferrox-cuda page, gqa_decode kernel source and the
 *     k_cache / v_cache shape in its doc comment); paged [pages, P, Hkv, D], the
 *     same order inside each page (reading: the page-level form of that layout).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

enum { OR_HND = 0, OR_NHD = 1 };

enum {
  OR_OK = 0,
  OR_BAD_ARG = 1,
  OR_BAD_INDPTR = 2,
  OR_BAD_INDEX = 3,
  OR_BAD_LAST_PAGE_LEN = 4,
  OR_NO_MEMORY = 5
};

/* ---------------------------------------------------------------- decoders */

double oracle_f16_to_f64(uint16_t h) {
  int neg = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return neg ? -v : v;
}

double oracle_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static size_t elem_size(int dtype) { return dtype == OR_F32 ? 4 : 2; }

static double load_elem(int dtype, const void *base, int64_t idx) {
  if (dtype == OR_F32) return (double)((const float *)base)[idx];
  uint16_t bits = ((const uint16_t *)base)[idx];
  return dtype == OR_F16 ? oracle_f16_to_f64(bits) : oracle_bf16_to_f64(bits);
}

/* ------------------------------------------------------------ page tables */

/* Checks the device-side contract of a page table.  Returns OR_OK or the first
 * violation found. */
int oracle_validate_table(int batch, int page_size, int num_total_pages,
                          int total_used_pages, const int32_t *indices,
                          const int32_t *indptr, const int32_t *last_page_len) {
  if (batch <= 0 || page_size <= 0 || num_total_pages <= 0 || total_used_pages < 0)
    return OR_BAD_ARG;
  if (indptr[0] != 0) return OR_BAD_INDPTR;
  for (int b = 0; b < batch; ++b)
    if (indptr[b + 1] < indptr[b]) return OR_BAD_INDPTR;
  if (indptr[batch] > total_used_pages) return OR_BAD_INDPTR;
  for (int i = 0; i < indptr[batch]; ++i)
    if (indices[i] < 0 || indices[i] >= num_total_pages) return OR_BAD_INDEX;
  for (int b = 0; b < batch; ++b)
    if (last_page_len[b] < 0 || last_page_len[b] > page_size) return OR_BAD_LAST_PAGE_LEN;
  return OR_OK;
}

/* L_b for every request (reading stated in the header). */
void oracle_seq_lens(int batch, int page_size, const int32_t *indptr,
                     const int32_t *last_page_len, int64_t *out_len) {
  for (int b = 0; b < batch; ++b) {
    int64_t n = (int64_t)indptr[b + 1] - indptr[b];
    out_len[b] = n == 0 ? 0 : (n - 1) * page_size + last_page_len[b];
  }
}

/* Element offset of row j of request b, kv head g, in a paged store laid out
 * [num_pages, num_kv_heads, page_size, head_dim] (OR_HND, heads-major inside a
 * page) or [num_pages, page_size, num_kv_heads, head_dim] (OR_NHD). */
static int64_t paged_row_offset(int layout, int num_kv_heads, int page_size, int head_dim,
                                const int32_t *indices, const int32_t *indptr, int b,
                                int g, int64_t j) {
  int64_t page = indices[indptr[b] + j / page_size];
  int64_t r = j % page_size;
  if (layout == OR_NHD) return ((page * page_size + r) * num_kv_heads + g) * head_dim;
  return ((page * num_kv_heads + g) * page_size + r) * head_dim;
}

/* Element offset of row j of kv head g in a contiguous cache of max_kv_len rows:
 * [num_kv_heads, max_kv_len, head_dim] (OR_HND) or [max_kv_len, num_kv_heads,
 * head_dim] (OR_NHD). */
static int64_t contig_row_offset(int layout, int num_kv_heads, int max_kv_len, int head_dim,
                                 int g, int64_t j) {
  if (layout == OR_NHD) return (j * num_kv_heads + g) * head_dim;
  return ((int64_t)g * max_kv_len + j) * head_dim;
}

/* Copies the page-table-resolved rows of K (or V), as raw element bits, into
 * out laid out [sum_b L_b, num_kv_heads, head_dim] (requests in order, rows in
 * order).  out must hold sum_b L_b * num_kv_heads * head_dim elements. */
int oracle_gather_paged(int dtype, int batch, int num_kv_heads, int head_dim,
                        int page_size, const void *data, const int32_t *indices,
                        const int32_t *indptr, const int32_t *last_page_len, void *out,
                        int layout) {
  if (layout != OR_HND && layout != OR_NHD) return OR_BAD_ARG;
  size_t es = elem_size(dtype);
  int64_t row_out = 0;
  for (int b = 0; b < batch; ++b) {
    int64_t n = (int64_t)indptr[b + 1] - indptr[b];
    int64_t L = n == 0 ? 0 : (n - 1) * page_size + last_page_len[b];
    for (int64_t j = 0; j < L; ++j, ++row_out) {
      for (int g = 0; g < num_kv_heads; ++g) {
        int64_t src = paged_row_offset(layout, num_kv_heads, page_size, head_dim, indices,
                                       indptr, b, g, j);
        int64_t dst = (row_out * num_kv_heads + g) * head_dim;
        memcpy((char *)out + dst * es, (const char *)data + src * es, head_dim * es);
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------ attention */

/* First row a query sees among L rows under a sliding window (0: no window). */
static int64_t window_start(int64_t L, int window) {
  return (window > 0 && L > window) ? L - window : 0;
}

/* Whether row bit `bit` of a custom mask keeps its row (NULL mask: every row). */
static int mask_keeps(const uint8_t *mask, int64_t bit) {
  return mask == NULL || ((mask[bit >> 3] >> (bit & 7)) & 1);
}

/* One query row against L explicit K/V rows given by element offsets into k and
 * v.  q_off is the element offset of the query row; row j's score gains
 * slope * dist[j] (its distance from the query's position).  Two-pass softmax
 * in f64.  o gets head_dim values; *lse the natural-log log-sum-exp. */
static void attend_rows(int dtype, int head_dim, double scale, double softcap, double slope,
                        const int64_t *dist, const void *q, int64_t q_off, const void *k,
                        const void *v, const int64_t *row_off, int64_t L, double *x, double *o,
                        double *lse) {
  for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
  if (L == 0) {
    *lse = -INFINITY;
    return;
  }
  /* scores */
  for (int64_t j = 0; j < L; ++j) {
    double dot = 0.0;
    for (int d = 0; d < head_dim; ++d)
      dot += load_elem(dtype, q, q_off + d) * load_elem(dtype, k, row_off[j] + d);
    x[j] = scale * dot + slope * (double)dist[j];
    if (softcap > 0.0) x[j] = softcap * tanh(x[j] / softcap);
  }
  /* pass 1: max */
  double M = x[0];
  for (int64_t j = 1; j < L; ++j)
    if (x[j] > M) M = x[j];
  /* pass 2: weights, normaliser, weighted V */
  double l = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    double w = exp(x[j] - M);
    l += w;
    for (int d = 0; d < head_dim; ++d) o[d] += w * load_elem(dtype, v, row_off[j] + d);
  }
  for (int d = 0; d < head_dim; ++d) o[d] /= l;
  *lse = M + log(l);
}

/* Paged decode.  q [batch, Hq, D], k/v [num_pages, Hkv, P, D] (OR_HND) or
 * [num_pages, P, Hkv, D] (OR_NHD) in dtype; outputs
 * o [batch, Hq, D] and lse [batch, Hq] in f64.  If n_sample > 0 only the listed
 * (sample_b[i], sample_h[i]) pairs are computed, into o[i*D ..] and lse[i].
 * threads <= 0 uses the OpenMP default. */
int oracle_decode_paged(int dtype, int batch, int num_qo_heads, int num_kv_heads,
                        int head_dim, int page_size, double scale, const void *q,
                        const void *k, const void *v, const int32_t *indices,
                        const int32_t *indptr, const int32_t *last_page_len, int n_sample,
                        const int32_t *sample_b, const int32_t *sample_h, double *o,
                        double *lse, int threads, int layout, int window, double softcap,
                        const double *alibi, const uint8_t *mask) {
  if (batch <= 0 || num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      page_size <= 0 || num_qo_heads % num_kv_heads != 0 ||
      (layout != OR_HND && layout != OR_NHD) || window < 0 || !(softcap >= 0.0))
    return OR_BAD_ARG;
  int group = num_qo_heads / num_kv_heads;
  int64_t n_items = n_sample > 0 ? n_sample : (int64_t)batch * num_qo_heads;
  /* rows_before[b] = L_0 + .. + L_{b-1}: where request b's mask bits start */
  int64_t *rows_before = (int64_t *)malloc(sizeof(int64_t) * (size_t)(batch + 1));
  if (!rows_before) return OR_NO_MEMORY;
  rows_before[0] = 0;
  for (int b = 0; b < batch; ++b) {
    int64_t n = (int64_t)indptr[b + 1] - indptr[b];
    rows_before[b + 1] = rows_before[b] + (n == 0 ? 0 : (n - 1) * page_size + last_page_len[b]);
  }
  int status = OR_OK;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
  for (int64_t it = 0; it < n_items; ++it) {
    int b = n_sample > 0 ? sample_b[it] : (int)(it / num_qo_heads);
    int h = n_sample > 0 ? sample_h[it] : (int)(it % num_qo_heads);
    int g = h / group;
    int64_t n = (int64_t)indptr[b + 1] - indptr[b];
    int64_t L = n == 0 ? 0 : (n - 1) * page_size + last_page_len[b];
    size_t cap = (size_t)(L > 0 ? L : 1);
    int64_t *row_off = (int64_t *)malloc(sizeof(int64_t) * cap);
    int64_t *dist = (int64_t *)malloc(sizeof(int64_t) * cap);
    double *x = (double *)malloc(sizeof(double) * cap);
    if (!row_off || !dist || !x) {
      status = OR_NO_MEMORY;
    } else {
      int64_t kept = 0;
      for (int64_t j = window_start(L, window); j < L; ++j) {
        if (!mask_keeps(mask, rows_before[b] + j)) continue;
        row_off[kept] = paged_row_offset(layout, num_kv_heads, page_size, head_dim, indices,
                                         indptr, b, g, j);
        dist[kept++] = j - (L - 1);
      }
      int64_t q_off = ((int64_t)b * num_qo_heads + h) * head_dim;
      attend_rows(dtype, head_dim, scale, softcap, alibi ? alibi[h] : 0.0, dist, q, q_off, k,
                  v, row_off, kept, x, o + it * head_dim, lse + it);
    }
    free(row_off);
    free(dist);
    free(x);
  }
  free(rows_before);
  return status;
}

/* Contiguous decode.  q [Hq, D], k/v [Hkv, max_kv_len, D] (OR_HND) or
 * [max_kv_len, Hkv, D] (OR_NHD); only rows
 * [0, valid_kv_len) take part (ferrum-kernels page, decode_attention argument
 * list).  o [Hq, D] and lse [Hq] in f64. */
int oracle_decode_contig(int dtype, int num_qo_heads, int num_kv_heads, int head_dim,
                         int max_kv_len, int valid_kv_len, double scale, const void *q,
                         const void *k, const void *v, double *o, double *lse,
                         int threads, int layout, int window, double softcap,
                         const double *alibi, const uint8_t *mask) {
  if (num_qo_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_kv_len < 0 ||
      valid_kv_len < 0 || valid_kv_len > max_kv_len || num_qo_heads % num_kv_heads != 0 ||
      (layout != OR_HND && layout != OR_NHD) || window < 0 || !(softcap >= 0.0))
    return OR_BAD_ARG;
  int group = num_qo_heads / num_kv_heads;
  int status = OR_OK;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
  for (int h = 0; h < num_qo_heads; ++h) {
    int g = h / group;
    int64_t L = valid_kv_len;
    size_t cap = (size_t)(L > 0 ? L : 1);
    int64_t *row_off = (int64_t *)malloc(sizeof(int64_t) * cap);
    int64_t *dist = (int64_t *)malloc(sizeof(int64_t) * cap);
    double *x = (double *)malloc(sizeof(double) * cap);
    if (!row_off || !dist || !x) {
      status = OR_NO_MEMORY;
    } else {
      int64_t kept = 0;
      for (int64_t j = window_start(L, window); j < L; ++j) {
        if (!mask_keeps(mask, j)) continue;
        row_off[kept] = contig_row_offset(layout, num_kv_heads, max_kv_len, head_dim, g, j);
        dist[kept++] = j - (L - 1);
      }
      attend_rows(dtype, head_dim, scale, softcap, alibi ? alibi[h] : 0.0, dist, q,
                  (int64_t)h * head_dim, k, v, row_off, kept, x, o + (int64_t)h * head_dim,
                  lse + h);
    }
    free(row_off);
    free(dist);
    free(x);
  }
  return status;
}

/* One query row (f64) against L explicit f64 K/V rows [L, D]: the partial that
 * a split of the KV range produces.  Same two-pass definition as above. */
void oracle_attend_f64(int head_dim, int64_t L, double scale, const double *q,
                       const double *k, const double *v, double *o, double *lse) {
  for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
  if (L <= 0) {
    *lse = -INFINITY;
    return;
  }
  double *x = (double *)malloc(sizeof(double) * (size_t)L);
  if (!x) {
    *lse = NAN;
    return;
  }
  for (int64_t j = 0; j < L; ++j) {
    double dot = 0.0;
    for (int d = 0; d < head_dim; ++d) dot += q[d] * k[j * head_dim + d];
    x[j] = scale * dot;
  }
  double M = x[0];
  for (int64_t j = 1; j < L; ++j)
    if (x[j] > M) M = x[j];
  double l = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    double w = exp(x[j] - M);
    l += w;
    for (int d = 0; d < head_dim; ++d) o[d] += w * v[j * head_dim + d];
  }
  for (int d = 0; d < head_dim; ++d) o[d] /= l;
  *lse = M + log(l);
  free(x);
}

/* Merge of S partial results (o_s normalised over its own rows, lse_s) of one
 * query row over a partition of its KV rows into the result over the union:
 *   lse = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) * o_s.
 * Evaluated with the max shift M = max_s lse_s.  Partials with lse_s = -inf
 * (empty parts) contribute nothing; if every part is empty, o = 0, lse = -inf. */
void oracle_merge(int head_dim, int n_parts, const double *o_parts, const double *lse_parts,
                  double *o, double *lse) {
  double M = -INFINITY;
  for (int s = 0; s < n_parts; ++s)
    if (lse_parts[s] > M) M = lse_parts[s];
  for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
  if (M == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  double sum = 0.0;
  for (int s = 0; s < n_parts; ++s) sum += exp(lse_parts[s] - M);
  double out_lse = M + log(sum);
  for (int s = 0; s < n_parts; ++s) {
    if (lse_parts[s] == -INFINITY) continue;
    double w = exp(lse_parts[s] - out_lse);
    for (int d = 0; d < head_dim; ++d) o[d] += w * o_parts[(int64_t)s * head_dim + d];
  }
  *lse = out_lse;
}

/* ------------------------------------------------------------ KV append */

/* Decode-time append of one new K (or V) row per request into a paged store
 * (baracuda-kernels page, "Companion plans": a plan that writes the new K/V
 * slices into the paged store at decode time; the page gives no signature).
 * Reading: the page table passed in already counts the new token, so request
 * b's new row is its last valid row, j = L_b - 1 (which lies in the
 * second-to-last page when last_page_len[b] = 0); a request with L_b = 0
 * receives nothing.  new_rows is [batch, Hkv, D]; data (layout as above) is
 * updated in place, nothing else in it changes. */
int oracle_append_paged(int dtype, int batch, int num_kv_heads, int head_dim, int page_size,
                        void *data, const int32_t *indices, const int32_t *indptr,
                        const int32_t *last_page_len, const void *new_rows, int layout) {
  if (batch <= 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0 ||
      (layout != OR_HND && layout != OR_NHD))
    return OR_BAD_ARG;
  size_t es = elem_size(dtype);
  for (int b = 0; b < batch; ++b) {
    int64_t n = (int64_t)indptr[b + 1] - indptr[b];
    int64_t L = n == 0 ? 0 : (n - 1) * page_size + last_page_len[b];
    if (L == 0) continue;
    for (int g = 0; g < num_kv_heads; ++g) {
      int64_t dst = paged_row_offset(layout, num_kv_heads, page_size, head_dim, indices, indptr,
                                     b, g, L - 1);
      int64_t src = ((int64_t)b * num_kv_heads + g) * head_dim;
      memcpy((char *)data + dst * es, (const char *)new_rows + src * es, head_dim * es);
    }
  }
  return OR_OK;
}
