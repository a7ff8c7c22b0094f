/* The float64 oracle (oracle/decode_ref.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer, on the CPU.  Linked with the oracle's source,
 * it calls every exported function on random small problems whose buffers
 * are allocated to exactly the sizes the functions are documented to read and
 * write -- every element type, both K/V layouts, page sizes 1..16, empty
 * requests and empty last pages, sliding windows, soft-caps, ALiBi slopes,
 * custom masks, the sampled mode, the contiguous cache, the append, the merge
 * and the attention over explicit rows -- and the table validator on broken
 * tables too.  An out-of-bounds access, a leak or undefined behaviour aborts
 * the run.  Test infrastructure only, like the oracle.  Prints "oracle driver
 * OK" and exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (oracle/decode_ref.c) */
int oracle_validate_table(int batch, int page_size, int num_total_pages, int total_used_pages,
                          const int32_t *indices, const int32_t *indptr,
                          const int32_t *last_page_len);
void oracle_seq_lens(int batch, int page_size, const int32_t *indptr,
                     const int32_t *last_page_len, int64_t *out_len);
int oracle_gather_paged(int dtype, int batch, int num_kv_heads, int head_dim, int page_size,
                        const void *data, const int32_t *indices, const int32_t *indptr,
                        const int32_t *last_page_len, void *out, int layout);
int oracle_decode_paged(int dtype, int batch, int num_qo_heads, int num_kv_heads, int head_dim,
                        int page_size, double scale, const void *q, const void *k,
                        const void *v, const int32_t *indices, const int32_t *indptr,
                        const int32_t *last_page_len, int n_sample, const int32_t *sample_b,
                        const int32_t *sample_h, double *o, double *lse, int threads,
                        int layout, int window, double softcap, const double *alibi,
                        const uint8_t *mask);
int oracle_decode_contig(int dtype, int num_qo_heads, int num_kv_heads, int head_dim,
                         int max_kv_len, int valid_kv_len, double scale, const void *q,
                         const void *k, const void *v, double *o, double *lse, int threads,
                         int layout, int window, double softcap, const double *alibi,
                         const uint8_t *mask);
void oracle_attend_f64(int head_dim, int64_t L, double scale, const double *q, const double *k,
                       const double *v, double *o, double *lse);
void oracle_merge(int head_dim, int n_parts, const double *o_parts, const double *lse_parts,
                  double *o, double *lse);
int oracle_append_paged(int dtype, int batch, int num_kv_heads, int head_dim, int page_size,
                        void *data, const int32_t *indices, const int32_t *indptr,
                        const int32_t *last_page_len, const void *new_rows, int layout);

static uint64_t g_state = 0x243F6A8885A308D3ull;

static uint64_t next_u64(void) { /* xorshift64* */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}

static int rand_int(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }

static double rand_unit(void) { return (double)(next_u64() >> 11) / 9007199254740992.0; }

static size_t elem_bytes(int dtype) { return dtype == 0 ? 4 : 2; }

/* n finite elements of modest magnitude, as raw bits of the element type */
static void *rand_elems(int dtype, size_t n) {
  void *p = malloc(n * elem_bytes(dtype) + 1);
  for (size_t i = 0; i < n; ++i) {
    if (dtype == 0) {
      ((float *)p)[i] = (float)(rand_unit() * 4.0 - 2.0);
    } else {
      const uint16_t sign = (uint16_t)((next_u64() & 1) << 15);
      const uint16_t mant = (uint16_t)(next_u64() & (dtype == 1 ? 0x3ff : 0x7f));
      const uint16_t ex = dtype == 1 ? (uint16_t)(rand_int(10, 16) << 10)
                                     : (uint16_t)(rand_int(122, 128) << 7);
      ((uint16_t *)p)[i] = (uint16_t)(sign | ex | mant);
    }
  }
  return p;
}

static int g_fail = 0;

static void expect(int ok, const char *what, int trial) {
  if (!ok && g_fail++ < 10) fprintf(stderr, "FAIL %s (trial %d)\n", what, trial);
}

static void paged_trial(int trial) {
  const int dtype = rand_int(0, 2), layout = rand_int(0, 1);
  const int batch = rand_int(1, 5), hkv = rand_int(1, 3), group = rand_int(1, 3);
  const int hq = hkv * group, d = (int[]){1, 2, 3, 8, 16}[rand_int(0, 4)];
  const int page = rand_int(1, 16);
  int32_t *indptr = malloc(sizeof(int32_t) * (batch + 1));
  int32_t *lpl = malloc(sizeof(int32_t) * batch);
  int used = 0;
  indptr[0] = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = rand_int(0, 3) == 0 ? 0 : rand_int(1, 40);
    int n = (L + page - 1) / page;
    int last = n ? L - (n - 1) * page : 0;
    if (L > 0 && L % page == 0 && rand_int(0, 2) == 0) { /* one more, empty page */
      ++n;
      last = 0;
    }
    lpl[b] = last;
    used += n;
    indptr[b + 1] = used;
  }
  const int pool = used + rand_int(1, 4);
  int32_t *indices = malloc(sizeof(int32_t) * (used + 1));
  int32_t *perm = malloc(sizeof(int32_t) * pool);
  for (int i = 0; i < pool; ++i) perm[i] = i;
  for (int i = pool - 1; i > 0; --i) {
    const int j = rand_int(0, i);
    const int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  memcpy(indices, perm, sizeof(int32_t) * used);
  expect(oracle_validate_table(batch, page, pool, used, indices, indptr, lpl) == 0,
         "valid table accepted", trial);
  int64_t *lens = malloc(sizeof(int64_t) * batch);
  oracle_seq_lens(batch, page, indptr, lpl, lens);
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) total += lens[b];

  const size_t pool_elems = (size_t)pool * hkv * page * d;
  void *k = rand_elems(dtype, pool_elems), *v = rand_elems(dtype, pool_elems);
  void *q = rand_elems(dtype, (size_t)batch * hq * d);
  const double scale = 0.05 + rand_unit();
  const int window = rand_int(0, 2) == 0 ? rand_int(1, 20) : 0;
  const double cap = rand_int(0, 2) == 0 ? 0.5 + 3.0 * rand_unit() : 0.0;
  double *alibi = NULL;
  if (rand_int(0, 1)) {
    alibi = malloc(sizeof(double) * hq);
    for (int h = 0; h < hq; ++h) alibi[h] = -0.5 + rand_unit();
  }
  uint8_t *mask = NULL;
  if (rand_int(0, 1)) {
    const size_t mb = (size_t)(total + 7) / 8 + (total == 0);
    mask = malloc(mb);
    for (size_t i = 0; i < mb; ++i) mask[i] = (uint8_t)next_u64();
  }
  /* whole output */
  double *o = malloc(sizeof(double) * (size_t)batch * hq * d);
  double *lse = malloc(sizeof(double) * (size_t)batch * hq);
  expect(oracle_decode_paged(dtype, batch, hq, hkv, d, page, scale, q, k, v, indices, indptr,
                             lpl, 0, NULL, NULL, o, lse, 2, layout, window, cap, alibi,
                             mask) == 0,
         "decode_paged", trial);
  /* sampled pairs */
  const int ns = rand_int(1, 6);
  int32_t *sb = malloc(sizeof(int32_t) * ns), *sh = malloc(sizeof(int32_t) * ns);
  for (int i = 0; i < ns; ++i) {
    sb[i] = rand_int(0, batch - 1);
    sh[i] = rand_int(0, hq - 1);
  }
  double *os = malloc(sizeof(double) * ns * d), *ls = malloc(sizeof(double) * ns);
  expect(oracle_decode_paged(dtype, batch, hq, hkv, d, page, scale, q, k, v, indices, indptr,
                             lpl, ns, sb, sh, os, ls, 1, layout, window, cap, alibi, mask) == 0,
         "decode_paged sampled", trial);
  for (int i = 0; i < ns; ++i)
    expect(ls[i] == lse[(size_t)sb[i] * hq + sh[i]] ||
               (isinf(ls[i]) && isinf(lse[(size_t)sb[i] * hq + sh[i]])),
           "sampled lse equals whole", trial);
  /* gather and append */
  void *g = malloc((size_t)(total ? total : 1) * hkv * d * elem_bytes(dtype));
  expect(oracle_gather_paged(dtype, batch, hkv, d, page, k, indices, indptr, lpl, g, layout) ==
             0,
         "gather", trial);
  void *rows = rand_elems(dtype, (size_t)batch * hkv * d);
  expect(oracle_append_paged(dtype, batch, hkv, d, page, k, indices, indptr, lpl, rows,
                             layout) == 0,
         "append", trial);
  /* broken tables: the validator reports them */
  if (batch > 1) {
    int32_t *bad = malloc(sizeof(int32_t) * (batch + 1));
    memcpy(bad, indptr, sizeof(int32_t) * (batch + 1));
    bad[1] = used + 5;
    expect(oracle_validate_table(batch, page, pool, used, indices, bad, lpl) != 0,
           "broken indptr rejected", trial);
    free(bad);
  }
  if (used > 0) {
    const int32_t keep = indices[0];
    indices[0] = pool;
    expect(oracle_validate_table(batch, page, pool, used, indices, indptr, lpl) != 0,
           "out-of-range page rejected", trial);
    indices[0] = keep;
  }
  free(indptr); free(lpl); free(indices); free(perm); free(lens); free(k); free(v); free(q);
  free(alibi); free(mask); free(o); free(lse); free(sb); free(sh); free(os); free(ls); free(g);
  free(rows);
}

static void contig_trial(int trial) {
  const int dtype = rand_int(0, 2), layout = rand_int(0, 1);
  const int hkv = rand_int(1, 3), hq = hkv * rand_int(1, 3), d = rand_int(1, 9);
  const int max_len = rand_int(1, 50), valid = rand_int(0, max_len);
  const size_t n = (size_t)hkv * max_len * d;
  void *k = rand_elems(dtype, n), *v = rand_elems(dtype, n), *q = rand_elems(dtype, (size_t)hq * d);
  uint8_t *mask = NULL;
  if (rand_int(0, 1)) {
    mask = malloc((size_t)(valid + 7) / 8 + 1);
    for (int i = 0; i < (valid + 7) / 8 + 1; ++i) mask[i] = (uint8_t)next_u64();
  }
  double *o = malloc(sizeof(double) * hq * d), *lse = malloc(sizeof(double) * hq);
  expect(oracle_decode_contig(dtype, hq, hkv, d, max_len, valid, 0.3, q, k, v, o, lse, 2, layout,
                              rand_int(0, 1) ? rand_int(1, 9) : 0,
                              rand_int(0, 1) ? 1.5 : 0.0, NULL, mask) == 0,
         "decode_contig", trial);
  free(k); free(v); free(q); free(mask); free(o); free(lse);
}

static void rows_trial(int trial) {
  const int d = rand_int(1, 16), L = rand_int(0, 30), S = rand_int(1, 6);
  double *q = malloc(sizeof(double) * d), *k = malloc(sizeof(double) * (L + 1) * d),
         *v = malloc(sizeof(double) * (L + 1) * d), *o = malloc(sizeof(double) * d), lse;
  for (int i = 0; i < d; ++i) q[i] = rand_unit() - 0.5;
  for (int i = 0; i < L * d; ++i) {
    k[i] = rand_unit() * 2.0 - 1.0;
    v[i] = rand_unit() * 2.0 - 1.0;
  }
  oracle_attend_f64(d, L, 0.7, q, k, v, o, &lse);
  expect(L > 0 ? isfinite(lse) : isinf(lse), "attend lse", trial);
  double *op = malloc(sizeof(double) * S * d), *lp = malloc(sizeof(double) * S);
  for (int s = 0; s < S; ++s) {
    lp[s] = rand_int(0, 3) == 0 ? -INFINITY : rand_unit() * 4.0 - 2.0;
    for (int i = 0; i < d; ++i) op[s * d + i] = rand_unit();
  }
  oracle_merge(d, S, op, lp, o, &lse);
  free(q); free(k); free(v); free(o); free(op); free(lp);
}

int main(void) {
  for (int t = 0; t < 3000; ++t) paged_trial(t);
  for (int t = 0; t < 2000; ++t) contig_trial(t);
  for (int t = 0; t < 2000; ++t) rows_trial(t);
  if (g_fail) {
    fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  printf("oracle driver OK\n");
  return 0;
}
