/*
 * Drives every entry point of the fp64 oracle (oracle/pkv_oracle.c) over the
 * pages' worked examples, random small cases and each error path, with every
 * buffer allocated at its exact size, so that an AddressSanitizer /
 * UndefinedBehaviorSanitizer build of the oracle reports any out-of-bounds
 * access, use of freed memory or undefined arithmetic.  Values are pinned by
 * the Python tests; this program only checks status codes and a few exact
 * results, and exits non-zero on the first surprise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int pkvo_decode(int dtype, const void* q, void* k_cache, void* v_cache,
                const int32_t* block_table, const int32_t* cache_seqlens, const void* k_new,
                const void* v_new, int batch, int Hq, int Hkv, int D, int num_blocks, int bs,
                int max_blocks_per_seq, double scale, const int32_t* seqs, int n_seqs,
                double* out, int n_threads);
int pkvo_varlen(int dtype, const void* q, const void* k, const void* v, const int32_t* cu_q,
                const int32_t* cu_k, int max_len_q, int max_len_k, int batch, int total_q,
                int total_k, int Hq, int Hkv, int D, double scale, const int32_t* rows,
                int n_rows, double* out, int n_threads);
int pkvo_cache_write(int dtype, const void* k, const void* v, const int32_t* cu,
                     const int32_t* start, void* k_cache, void* v_cache,
                     const int32_t* block_table, int batch, int total, int Hkv, int D,
                     int num_blocks, int bs, int max_blocks_per_seq);
int pkvo_varlen_paged(int dtype, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* cu_q, const int32_t* seqlens_k,
                      int max_len_q, int max_len_k, int batch, int total_q, int Hq, int Hkv,
                      int D, int num_blocks, int bs, int max_blocks_per_seq, double scale,
                      const int32_t* rows, int n_rows, double* out, int n_threads);
void pkvo_cu_from_lengths(const int32_t* lengths, int batch, int32_t* cu);
int pkvo_request_index(const int32_t* cu, int batch, int total, int32_t* req);
int pkvo_locate(const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                int block_size, int seq, int64_t t, int32_t* where3);
void pkvo_partial(int n, const double* s, const double* vals, int d, double* m_out,
                  double* l_out, double* acc_out);
void pkvo_merge2(double m1, double l1, const double* a1, double m2, double l2, const double* a2,
                 int d, double* m_out, double* l_out, double* a_out);
void pkvo_finalize(double l, const double* acc, int d, double* out);
int pkvo_max_threads(void);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(rng_state >> 33);
}
static float rndf(void) { return ((float)(rnd() % 20001) - 10000.f) / 5000.f; }

/* n elements of dtype 0 (fp32) or 1 (bf16 bit patterns), exact size */
static void* rand_buf(int dtype, size_t n) {
  if (dtype == 0) {
    float* p = (float*)malloc(n * sizeof(float) + (n == 0));
    for (size_t i = 0; i < n; ++i) p[i] = rndf();
    return p;
  }
  uint16_t* p = (uint16_t*)malloc(n * sizeof(uint16_t) + (n == 0));
  for (size_t i = 0; i < n; ++i) {
    float f = rndf();
    uint32_t b;
    memcpy(&b, &f, 4);
    p[i] = (uint16_t)(b >> 16);
  }
  return p;
}

static int failures = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static void decode_cases(void) {
  /* HF page decode example: cached 30/32/70, block size 32, append */
  {
    const int B = 3, H = 4, D = 64, bs = 32, NB = 8, MB = 4;
    const int32_t table[12] = {2, -1, -1, -1, 0, 1, -1, -1, 3, 5, 6, -1};
    const int32_t lens[3] = {30, 32, 70};
    float* q = rand_buf(0, (size_t)B * H * D);
    float* kc = rand_buf(0, (size_t)NB * bs * H * D);
    float* vc = rand_buf(0, (size_t)NB * bs * H * D);
    float* kn = rand_buf(0, (size_t)B * H * D);
    float* vn = rand_buf(0, (size_t)B * H * D);
    double* out = malloc(sizeof(double) * B * H * D);
    EXPECT(pkvo_decode(0, q, kc, vc, table, lens, kn, vn, B, H, H, D, NB, bs, MB, 0.125, NULL, 0,
                       out, 0) == 0);
    EXPECT(memcmp(kc + ((size_t)2 * bs + 30) * H * D, kn, sizeof(float) * H * D) == 0);
    EXPECT(memcmp(kc + ((size_t)1 * bs + 0) * H * D, kn + H * D, sizeof(float) * H * D) == 0);
    EXPECT(memcmp(kc + ((size_t)6 * bs + 6) * H * D, kn + 2 * H * D, sizeof(float) * H * D) == 0);
    /* a needed entry of -1 (sequence 1 at 64 cached tokens + 1 needs block 2) */
    const int32_t lens2[3] = {30, 64, 70};
    EXPECT(pkvo_decode(0, q, kc, vc, table, lens2, kn, vn, B, H, H, D, NB, bs, MB, 0.125, NULL, 0,
                       out, 0) == 2);
    /* past the table row, negative length */
    const int32_t lens3[3] = {30, 32, 129};
    EXPECT(pkvo_decode(0, q, kc, vc, table, lens3, NULL, NULL, B, H, H, D, NB, bs, MB, 0.125,
                       NULL, 0, out, 0) == 3);
    const int32_t lens4[3] = {30, -1, 70};
    EXPECT(pkvo_decode(0, q, kc, vc, table, lens4, NULL, NULL, B, H, H, D, NB, bs, MB, 0.125,
                       NULL, 0, out, 0) == 4);
    free(q); free(kc); free(vc); free(kn); free(vn); free(out);
  }
  /* random bf16 GQA batches, with and without append, a subset of sequences */
  for (int trial = 0; trial < 6; ++trial) {
    const int B = 1 + (int)(rnd() % 6), Hkv = 1 + (int)(rnd() % 3), G = 1 + (int)(rnd() % 4);
    const int H = Hkv * G, D = (trial & 1) ? 8 : 5, bs = (trial & 2) ? 4 : 16;
    const int append = trial % 3 != 0;
    const int MB = 6, NB = B * MB + 2;
    int32_t* table = malloc(sizeof(int32_t) * B * MB);
    int32_t* lens = malloc(sizeof(int32_t) * B);
    for (int i = 0; i < B; ++i) {
      lens[i] = (int)(rnd() % (unsigned)(MB * bs - append + 1));
      for (int j = 0; j < MB; ++j) table[i * MB + j] = (i * MB + j + 3 * trial) % NB;
    }
    lens[0] = 0;
    void* q = rand_buf(1, (size_t)B * H * D);
    void* kc = rand_buf(1, (size_t)NB * bs * Hkv * D);
    void* vc = rand_buf(1, (size_t)NB * bs * Hkv * D);
    void* kn = append ? rand_buf(1, (size_t)B * Hkv * D) : NULL;
    void* vn = append ? rand_buf(1, (size_t)B * Hkv * D) : NULL;
    int32_t seqs[2] = {B - 1, 0};
    double* out = malloc(sizeof(double) * B * H * D);
    EXPECT(pkvo_decode(1, q, kc, vc, table, lens, kn, vn, B, H, Hkv, D, NB, bs, MB, 0.4, NULL, 0,
                       out, 0) == 0);
    if (!append)
      for (int e = 0; e < H * D; ++e) EXPECT(out[e] == 0.0); /* no key: zeros */
    EXPECT(pkvo_decode(1, q, kc, vc, table, lens, kn, vn, B, H, Hkv, D, NB, bs, MB, 0.4, seqs, 2,
                       out, 2) == 0);
    free(table); free(lens); free(q); free(kc); free(vc); free(kn); free(vn); free(out);
  }
}

static void varlen_cases(void) {
  /* HF page varlen example: q lengths 10/3/1, k lengths 0/1/7 */
  const int32_t lq[3] = {10, 3, 1}, lk[3] = {0, 1, 7};
  int32_t cq[4], ck[4], req[14];
  pkvo_cu_from_lengths(lq, 3, cq);
  pkvo_cu_from_lengths(lk, 3, ck);
  EXPECT(cq[3] == 14 && ck[3] == 8 && ck[1] == 0 && ck[2] == 1);
  EXPECT(pkvo_request_index(cq, 3, 14, req) == 0 && req[0] == 0 && req[12] == 1 && req[13] == 2);
  const int Hq = 8, Hkv = 2, D = 6;
  void* q = rand_buf(1, (size_t)14 * Hq * D);
  void* k = rand_buf(1, (size_t)8 * Hkv * D);
  void* v = rand_buf(1, (size_t)8 * Hkv * D);
  double* out = malloc(sizeof(double) * 14 * Hq * D);
  EXPECT(pkvo_varlen(1, q, k, v, cq, ck, 10, 7, 3, 14, 8, Hq, Hkv, D, 0.3, NULL, 0, out, 0) == 0);
  for (int e = 0; e < 10 * Hq * D; ++e) EXPECT(out[e] == 0.0);
  const int32_t rows[3] = {13, 0, 11};
  EXPECT(pkvo_varlen(1, q, k, v, cq, ck, 10, 7, 3, 14, 8, Hq, Hkv, D, 0.3, rows, 3, out, 1) == 0);
  EXPECT(pkvo_varlen(1, q, k, v, cq, ck, 9, 7, 3, 14, 8, Hq, Hkv, D, 0.3, NULL, 0, out, 0) == 6);
  int32_t bad[4] = {0, 5, 3, 14};
  EXPECT(pkvo_varlen(1, q, k, v, bad, ck, 10, 7, 3, 14, 8, Hq, Hkv, D, 0.3, NULL, 0, out, 0) == 5);
  const int32_t badrow[1] = {14};
  EXPECT(pkvo_varlen(1, q, k, v, cq, ck, 10, 7, 3, 14, 8, Hq, Hkv, D, 0.3, badrow, 1, out, 0) == 1);
  free(q); free(k); free(v); free(out);
}

static void paged_prefill_cases(void) {
  /* three requests: cached prefixes 5 / 0 / 17, new rows 3 / 0 / 20, blocks of 4 */
  const int B = 3, Hq = 4, Hkv = 2, D = 3, bs = 4, MB = 10, NB = 30;
  const int32_t start[3] = {5, 0, 17}, newl[3] = {3, 0, 20};
  int32_t cu[4], table[30], seqlens[3];
  pkvo_cu_from_lengths(newl, B, cu);
  for (int i = 0; i < B * MB; ++i) table[i] = (7 * i + 1) % NB;
  for (int b = 0; b < B; ++b) seqlens[b] = start[b] + newl[b];
  const int total = cu[B];
  void* kn = rand_buf(0, (size_t)total * Hkv * D);
  void* vn = rand_buf(0, (size_t)total * Hkv * D);
  void* kc = rand_buf(0, (size_t)NB * bs * Hkv * D);
  void* vc = rand_buf(0, (size_t)NB * bs * Hkv * D);
  EXPECT(pkvo_cache_write(0, kn, vn, cu, start, kc, vc, table, B, total, Hkv, D, NB, bs, MB) == 0);
  void* q = rand_buf(0, (size_t)total * Hq * D);
  double* out = malloc(sizeof(double) * total * Hq * D);
  EXPECT(pkvo_varlen_paged(0, q, kc, vc, table, cu, seqlens, 20, 37, B, total, Hq, Hkv, D, NB, bs,
                           MB, 0.5, NULL, 0, out, 0) == 0);
  const int32_t past[3] = {5, 0, 40}; /* 40 + 20 tokens > 10 blocks of 4 */
  EXPECT(pkvo_cache_write(0, kn, vn, cu, past, kc, vc, table, B, total, Hkv, D, NB, bs, MB) == 3);
  int32_t hole[30];
  memcpy(hole, table, sizeof hole);
  hole[2 * MB + 5] = -1;
  EXPECT(pkvo_cache_write(0, kn, vn, cu, start, kc, vc, hole, B, total, Hkv, D, NB, bs, MB) == 2);
  EXPECT(pkvo_varlen_paged(0, q, kc, vc, hole, cu, seqlens, 20, 37, B, total, Hq, Hkv, D, NB, bs,
                           MB, 0.5, NULL, 0, out, 0) == 2);
  free(kn); free(vn); free(kc); free(vc); free(q); free(out);
}

static void index_and_merge_cases(void) {
  /* notes' 60-token sequence on blocks 7, 1, 12, 4 of 16 tokens */
  const int32_t row[4] = {7, 1, 12, 4};
  int32_t w[3];
  EXPECT(pkvo_locate(row, 4, 13, 16, 0, 59, w) == 0 && w[0] == 3 && w[1] == 11 && w[2] == 4);
  EXPECT(pkvo_locate(row, 4, 13, 16, 0, 64, w) == 3);
  EXPECT(pkvo_locate(row, 4, 12, 16, 0, 40, w) == 2);
  EXPECT(pkvo_locate(row, 4, 13, 16, 0, -1, w) == 3);
  /* partial / merge / finalize, including the empty run */
  double s[5] = {0.5, -1.0, 2.0, 0.0, 1.0}, vals[10];
  for (int i = 0; i < 10; ++i) vals[i] = i;
  double m1, l1, a1[2], m2, l2, a2[2], m, l, a[2], o[2];
  pkvo_partial(2, s, vals, 2, &m1, &l1, a1);
  pkvo_partial(3, s + 2, vals + 4, 2, &m2, &l2, a2);
  pkvo_merge2(m1, l1, a1, m2, l2, a2, 2, &m, &l, a);
  pkvo_finalize(l, a, 2, o);
  EXPECT(m == 2.0 && o[0] > 0.0);
  pkvo_partial(0, s, vals, 2, &m1, &l1, a1);
  EXPECT(isinf(m1) && m1 < 0 && l1 == 0.0);
  pkvo_merge2(m1, l1, a1, m1, l1, a1, 2, &m, &l, a);
  pkvo_finalize(l, a, 2, o);
  EXPECT(l == 0.0 && o[0] == 0.0 && o[1] == 0.0);
  EXPECT(pkvo_max_threads() >= 1);
}

int main(void) {
  decode_cases();
  varlen_cases();
  paged_prefill_cases();
  index_and_merge_cases();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("oracle driver ok\n");
  return 0;
}
