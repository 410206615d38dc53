/*
 * pkv_oracle.c -- plain fp64 CPU oracle for paged attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * What it computes (sources are the web pages this project follows):
 *
 *  - "39 · PagedAttention" (inference-notes), section 1: for one new decode
 *    token, its query is dotted with the key of every earlier token, one
 *    softmax turns those scores into weights summing to 1, and the output is
 *    the weight-sum of the value vectors.  Section 2 and the "Quan trọng"
 *    box: the paged version is exactly that, only the read addresses go
 *    through the block table.  The section-2 recipe is followed literally:
 *    walk the logical blocks in order to get every score, apply a single
 *    softmax over all of them, then walk the blocks again to sum the
 *    weighted values.
 *  - Same page, section 3: two partial results (max score m, sum of
 *    exponentials l) merge as m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m).
 *    The page gives only m and l; the unnormalised value sum is scaled by the
 *    same factor as l (the only reading under which the merged result is one
 *    softmax).
 *  - HF Transformers "paged attention" page, section "Jalur decode": the
 *    block table has shape (batch_size, max_blocks_per_seq), each row lists
 *    the physical cache blocks of one request, -1 marks an unallocated
 *    entry, cache_seqlens holds each sequence's cached length, one query
 *    token per sequence, and the cache is updated in place.  Section "Jalur
 *    Varlen": packed sequences delimited by the cumulative lengths
 *    cu_seq_lens_q / cu_seq_lens_k, bounded by max_length_q / max_length_k;
 *    its cache-behaviour note: that kernel cannot reach the paged cache, so
 *    the cache is written (and read) around it by a separate update.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - cache_seqlens counts tokens cached BEFORE the call; when new K/V are
 *    given they are written at slot cache_seqlens[i] and attended too.
 *  - Cache layout [num_blocks, block_size, num_kv_heads, head_dim], K and V
 *    in separate pools; packed layout [total, heads, head_dim].
 *  - Grouped heads: q head h reads kv head h / (num_heads / num_kv_heads).
 *  - A sequence with no key at all outputs zeros.
 *  - Inputs are fp32 or bf16 and are widened exactly to fp64; all
 *    arithmetic is fp64; the output is fp64.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (see oracle/build.py).  OpenMP only
 * spreads independent (sequence, head) or (row, head) units over threads; the
 * arithmetic inside a unit is a fixed sequential order, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { PKVO_F32 = 0, PKVO_BF16 = 1 };

enum {
  PKVO_OK = 0,
  PKVO_ERR_ARGS = 1,        /* bad scalar argument */
  PKVO_ERR_BLOCK = 2,       /* a needed block_table entry is -1 or >= num_blocks */
  PKVO_ERR_TABLE_SPAN = 3,  /* a needed logical block index is >= max_blocks_per_seq */
  PKVO_ERR_SEQLEN = 4,      /* negative cache_seqlens */
  PKVO_ERR_CU = 5,          /* cu_seq_lens not starting at 0 / decreasing / wrong total */
  PKVO_ERR_MAXLEN = 6       /* a length exceeds max_length_q or max_length_k */
};

/* Exact widening of one stored element to fp64.  A bf16 value is the upper
 * 16 bits of an IEEE binary32 value. */
static double widen(int dtype, const void* base, int64_t idx) {
  if (dtype == PKVO_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t elem_size(int dtype) { return dtype == PKVO_F32 ? 4 : 2; }

/* ---------------------------------------------------------------- indexing */

/* Exclusive prefix sum of per-request lengths: cu[0] = 0, cu[b+1] = cu[b] +
 * len[b] (HF page, "Jalur Varlen" example). */
void pkvo_cu_from_lengths(const int32_t* lengths, int batch, int32_t* cu) {
  cu[0] = 0;
  for (int b = 0; b < batch; ++b) cu[b + 1] = cu[b] + lengths[b];
}

/* The request each packed token belongs to: token r is in request b when
 * cu[b] <= r < cu[b+1] (HF page, "Jalur Varlen" example).  Returns 0, or
 * PKVO_ERR_CU when cu is not a valid cumulative array for `total` tokens. */
int pkvo_request_index(const int32_t* cu, int batch, int total, int32_t* req) {
  if (cu[0] != 0 || cu[batch] != total) return PKVO_ERR_CU;
  for (int b = 0; b < batch; ++b)
    if (cu[b + 1] < cu[b]) return PKVO_ERR_CU;
  for (int b = 0; b < batch; ++b)
    for (int r = cu[b]; r < cu[b + 1]; ++r) req[r] = b;
  return PKVO_OK;
}

/* Where logical token t of sequence i lives: logical block t / block_size,
 * offset t mod block_size, physical block block_table[i][t / block_size]
 * (HF page "Jalur decode" example; inference-notes section 2).  Writes
 * (logical block, offset, physical block).  Returns PKVO_ERR_TABLE_SPAN if the
 * logical block is past the table row, PKVO_ERR_BLOCK if the entry is -1 or
 * out of the pool. */
int pkvo_locate(const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                int block_size, int seq, int64_t t, int32_t* where3) {
  int64_t j = t / block_size;
  int64_t o = t % block_size;
  if (t < 0 || j >= max_blocks_per_seq) return PKVO_ERR_TABLE_SPAN;
  int32_t pb = block_table[(int64_t)seq * max_blocks_per_seq + j];
  where3[0] = (int32_t)j;
  where3[1] = (int32_t)o;
  where3[2] = pb;
  if (pb < 0 || pb >= num_blocks) return PKVO_ERR_BLOCK;
  return PKVO_OK;
}

/* ---------------------------------------------------------- softmax pieces */

/* Partial softmax state of a run of scores s[0..n) with value rows
 * val(t)[0..d): m = max s, l = sum e^(s - m), acc = sum e^(s - m) val(t).
 * n = 0 gives the identity (-inf, 0, 0).  Used by the merge-law checks. */
void pkvo_partial(int n, const double* s, const double* vals, int d,
                  double* m_out, double* l_out, double* acc_out) {
  double m = -INFINITY;
  for (int t = 0; t < n; ++t)
    if (s[t] > m) m = s[t];
  double l = 0.0;
  for (int c = 0; c < d; ++c) acc_out[c] = 0.0;
  if (n > 0) {
    for (int t = 0; t < n; ++t) {
      double w = exp(s[t] - m);
      l += w;
      for (int c = 0; c < d; ++c) acc_out[c] += w * vals[(int64_t)t * d + c];
    }
  }
  *m_out = m;
  *l_out = l;
}

/* Merge of two partial states (inference-notes section 3):
 *   m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m), acc likewise.
 * e^(-inf - m) is taken as 0, so the identity (-inf, 0, 0) merges to the
 * other operand and identity with identity stays the identity. */
void pkvo_merge2(double m1, double l1, const double* a1,
                 double m2, double l2, const double* a2, int d,
                 double* m_out, double* l_out, double* acc_out) {
  double m = m1 > m2 ? m1 : m2;
  double f1 = (m1 == -INFINITY) ? 0.0 : exp(m1 - m);
  double f2 = (m2 == -INFINITY) ? 0.0 : exp(m2 - m);
  *m_out = m;
  *l_out = l1 * f1 + l2 * f2;
  for (int c = 0; c < d; ++c) acc_out[c] = a1[c] * f1 + a2[c] * f2;
}

/* out = acc / l, or zeros when l = 0 (no key at all). */
void pkvo_finalize(double l, const double* acc, int d, double* out) {
  for (int c = 0; c < d; ++c) out[c] = (l > 0.0) ? acc[c] / l : 0.0;
}

/* ------------------------------------------------------------------ decode */

/* One (sequence, q head): the three-step recipe of inference-notes section 2
 * over logical tokens 0..len-1, reading K and V through the table row.
 * Every needed table entry has been validated by the caller. */
static void decode_one(int dtype, const void* q, const void* kc, const void* vc,
                       const int32_t* row, int len, int seq, int h, int G,
                       int Hq, int Hkv, int D, int bs, double scale,
                       double* s, double* out) {
  const int g = h / G;
  const int64_t qoff = ((int64_t)seq * Hq + h) * D;
  if (len == 0) {
    for (int c = 0; c < D; ++c) out[c] = 0.0;
    return;
  }
  /* step 1: walk the logical blocks in order, one score per token */
  const int nblk = (len + bs - 1) / bs;
  for (int j = 0; j < nblk; ++j) {
    const int64_t pb = row[j];
    for (int u = 0; u < bs && j * bs + u < len; ++u) {
      const int64_t koff = ((pb * bs + u) * Hkv + g) * D;
      double dot = 0.0;
      for (int c = 0; c < D; ++c) dot += widen(dtype, q, qoff + c) * widen(dtype, kc, koff + c);
      s[j * bs + u] = scale * dot;
    }
  }
  /* step 2: one softmax over all scores */
  double m = -INFINITY;
  for (int t = 0; t < len; ++t)
    if (s[t] > m) m = s[t];
  double l = 0.0;
  for (int t = 0; t < len; ++t) {
    s[t] = exp(s[t] - m);
    l += s[t];
  }
  /* step 3: walk the blocks again, summing weighted values */
  for (int c = 0; c < D; ++c) out[c] = 0.0;
  for (int j = 0; j < nblk; ++j) {
    const int64_t pb = row[j];
    for (int u = 0; u < bs && j * bs + u < len; ++u) {
      const int64_t voff = ((pb * bs + u) * Hkv + g) * D;
      const double w = s[j * bs + u];
      for (int c = 0; c < D; ++c) out[c] += w * widen(dtype, vc, voff + c);
    }
  }
  for (int c = 0; c < D; ++c) out[c] /= l;
}

/*
 * Decode attention over a paged cache, with optional in-place append.
 *
 *   q            [batch, 1, Hq, D]                    dtype
 *   k_cache      [num_blocks, bs, Hkv, D]             dtype, host copy, MUTATED by the append
 *   v_cache      same
 *   block_table  [batch, max_blocks_per_seq] int32, -1 = unallocated
 *   cache_seqlens[batch] int32, tokens cached before this call
 *   k_new, v_new [batch, 1, Hkv, D] or both NULL
 *   seqs         sequences whose output is wanted (NULL = all, in order)
 *   out          [n_eval, Hq, D] fp64
 *
 * Step order: (1) every sequence's new K/V row is written at slot
 * cache_seqlens[i] (logical block cache_seqlens[i] / bs, offset
 * cache_seqlens[i] mod bs, physical block from the table); (2) each wanted
 * sequence attends its cache_seqlens[i] (+1 with an append) tokens.
 * Returns PKVO_OK or the first error found (nothing is written when the
 * arguments or the table are bad).
 */
int pkvo_decode(int dtype, const void* q, void* k_cache, void* v_cache,
                const int32_t* block_table, const int32_t* cache_seqlens,
                const void* k_new, const void* v_new,
                int batch, int Hq, int Hkv, int D, int num_blocks, int bs,
                int max_blocks_per_seq, double scale,
                const int32_t* seqs, int n_seqs, double* out, int n_threads) {
  if (batch < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || Hq % Hkv != 0 || (dtype != PKVO_F32 && dtype != PKVO_BF16) ||
      ((k_new == NULL) != (v_new == NULL)))
    return PKVO_ERR_ARGS;
  const int append = k_new != NULL;
  const int G = Hq / Hkv;
  const size_t esz = elem_size(dtype);
  const int n_eval = seqs ? n_seqs : batch;

  /* validate every table entry a wanted or appending sequence needs */
  for (int i = 0; i < batch; ++i) {
    const int len = cache_seqlens[i];
    if (len < 0) return PKVO_ERR_SEQLEN;
    const int lenp = len + append;
    const int nblk = (lenp + bs - 1) / bs;
    if (nblk > max_blocks_per_seq) return PKVO_ERR_TABLE_SPAN;
    for (int j = 0; j < nblk; ++j) {
      const int32_t pb = block_table[(int64_t)i * max_blocks_per_seq + j];
      if (pb < 0 || pb >= num_blocks) return PKVO_ERR_BLOCK;
    }
  }
  for (int e = 0; e < n_eval; ++e)
    if (seqs && (seqs[e] < 0 || seqs[e] >= batch)) return PKVO_ERR_ARGS;

  /* (1) in-place append: a byte copy of the new row into its slot */
  if (append) {
    const size_t row_bytes = (size_t)Hkv * D * esz;
    for (int i = 0; i < batch; ++i) {
      int32_t w[3];
      int rc = pkvo_locate(block_table, max_blocks_per_seq, num_blocks, bs, i,
                           cache_seqlens[i], w);
      if (rc) return rc;
      const int64_t slot = (int64_t)w[2] * bs + w[1];
      memcpy((char*)k_cache + slot * row_bytes, (const char*)k_new + (int64_t)i * row_bytes, row_bytes);
      memcpy((char*)v_cache + slot * row_bytes, (const char*)v_new + (int64_t)i * row_bytes, row_bytes);
    }
  }

  /* (2) attention for every wanted (sequence, head) */
  int maxlen = 0;
  for (int e = 0; e < n_eval; ++e) {
    const int i = seqs ? seqs[e] : e;
    if (cache_seqlens[i] + append > maxlen) maxlen = cache_seqlens[i] + append;
  }
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
  const int64_t units = (int64_t)n_eval * Hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t uidx = 0; uidx < units; ++uidx) {
      const int e = (int)(uidx / Hq), h = (int)(uidx % Hq);
      const int i = seqs ? seqs[e] : e;
      decode_one(dtype, q, k_cache, v_cache, block_table + (int64_t)i * max_blocks_per_seq,
                 cache_seqlens[i] + append, i, h, G, Hq, Hkv, D, bs, scale, s,
                 out + ((int64_t)e * Hq + h) * D);
    }
    free(s);
  }
  return PKVO_OK;
}

/* ------------------------------------------------------------------ varlen */

/*
 * Attention over packed variable-length sequences, no mask: every query row
 * of request b attends every key row of request b.
 *
 *   q    [total_q, Hq, D], k/v [total_k, Hkv, D]  (the leading 1 is dropped)
 *   cu_q [batch+1], cu_k [batch+1] int32
 *   rows q rows whose output is wanted (NULL = all)
 *   out  [n_eval, Hq, D] fp64
 */
int pkvo_varlen(int dtype, const void* q, const void* k, const void* v,
                const int32_t* cu_q, const int32_t* cu_k, int max_len_q, int max_len_k,
                int batch, int total_q, int total_k, int Hq, int Hkv, int D, double scale,
                const int32_t* rows, int n_rows, double* out, int n_threads) {
  if (batch < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 ||
      (dtype != PKVO_F32 && dtype != PKVO_BF16))
    return PKVO_ERR_ARGS;
  if (cu_q[0] != 0 || cu_k[0] != 0 || cu_q[batch] != total_q || cu_k[batch] != total_k)
    return PKVO_ERR_CU;
  for (int b = 0; b < batch; ++b) {
    const int lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
    if (lq < 0 || lk < 0) return PKVO_ERR_CU;
    if (lq > max_len_q || lk > max_len_k) return PKVO_ERR_MAXLEN;
  }
  const int n_eval = rows ? n_rows : total_q;
  for (int e = 0; e < n_eval; ++e)
    if (rows && (rows[e] < 0 || rows[e] >= total_q)) return PKVO_ERR_ARGS;
  int32_t* req = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total_q > 0 ? total_q : 1));
  int rc = pkvo_request_index(cu_q, batch, total_q, req);
  if (rc) {
    free(req);
    return rc;
  }
  const int G = Hq / Hkv;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
  const int64_t units = (int64_t)n_eval * Hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_len_k > 0 ? max_len_k : 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t uidx = 0; uidx < units; ++uidx) {
      const int e = (int)(uidx / Hq), h = (int)(uidx % Hq);
      const int r = rows ? rows[e] : e;
      const int b = req[r];
      const int g = h / G;
      const int c0 = cu_k[b], n = cu_k[b + 1] - cu_k[b];
      double* o = out + ((int64_t)e * Hq + h) * D;
      const int64_t qoff = ((int64_t)r * Hq + h) * D;
      if (n == 0) {
        for (int c = 0; c < D; ++c) o[c] = 0.0;
        continue;
      }
      for (int t = 0; t < n; ++t) {
        const int64_t koff = ((int64_t)(c0 + t) * Hkv + g) * D;
        double dot = 0.0;
        for (int c = 0; c < D; ++c) dot += widen(dtype, q, qoff + c) * widen(dtype, k, koff + c);
        s[t] = scale * dot;
      }
      double m = -INFINITY;
      for (int t = 0; t < n; ++t)
        if (s[t] > m) m = s[t];
      double l = 0.0;
      for (int t = 0; t < n; ++t) {
        s[t] = exp(s[t] - m);
        l += s[t];
      }
      for (int c = 0; c < D; ++c) o[c] = 0.0;
      for (int t = 0; t < n; ++t) {
        const int64_t voff = ((int64_t)(c0 + t) * Hkv + g) * D;
        for (int c = 0; c < D; ++c) o[c] += s[t] * widen(dtype, v, voff + c);
      }
      for (int c = 0; c < D; ++c) o[c] /= l;
    }
    free(s);
  }
  free(req);
  return PKVO_OK;
}

/* -------------------------------------------------------- paged prefill */

/*
 * Writing packed rows into the paged cache.  The HF page, section "Jalur
 * Varlen", cache behaviour: the varlen kernel cannot reach the paged cache,
 * so new rows are written into it by a separate update.  Row cu[b] + i of
 * request b is token start[b] + i of sequence b and goes to slot
 * (block_table[b][p / bs], p mod bs), p = start[b] + i -- the same address
 * rule as the decode append ("Jalur decode"), applied to every row.  A byte
 * copy of the Hkv * D row, K and V alike.
 *
 *   k, v         [total, Hkv, D] dtype (the leading 1 is dropped)
 *   cu           [batch+1] int32, start [batch] int32 (>= 0)
 *   k_cache, v_cache [num_blocks, bs, Hkv, D], host copies, MUTATED
 *
 * Every row is located first; on any error nothing is written.
 */
int pkvo_cache_write(int dtype, const void* k, const void* v, const int32_t* cu,
                     const int32_t* start, void* k_cache, void* v_cache,
                     const int32_t* block_table, int batch, int total, int Hkv, int D,
                     int num_blocks, int bs, int max_blocks_per_seq) {
  if (batch < 0 || total < 0 || Hkv <= 0 || D <= 0 || bs <= 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || (dtype != PKVO_F32 && dtype != PKVO_BF16))
    return PKVO_ERR_ARGS;
  if (cu[0] != 0 || cu[batch] != total) return PKVO_ERR_CU;
  for (int b = 0; b < batch; ++b) {
    if (cu[b + 1] < cu[b]) return PKVO_ERR_CU;
    if (start[b] < 0) return PKVO_ERR_SEQLEN;
    for (int i = 0; i < cu[b + 1] - cu[b]; ++i) {
      int32_t w[3];
      const int rc = pkvo_locate(block_table, max_blocks_per_seq, num_blocks, bs, b,
                                 start[b] + i, w);
      if (rc) return rc;
    }
  }
  const size_t row_bytes = (size_t)Hkv * D * elem_size(dtype);
  for (int b = 0; b < batch; ++b)
    for (int i = 0; i < cu[b + 1] - cu[b]; ++i) {
      int32_t w[3] = {0, 0, 0};  /* every slot was located above */
      pkvo_locate(block_table, max_blocks_per_seq, num_blocks, bs, b, start[b] + i, w);
      const int64_t slot = (int64_t)w[2] * bs + w[1];
      const int64_t r = cu[b] + i;
      memcpy((char*)k_cache + slot * row_bytes, (const char*)k + r * row_bytes, row_bytes);
      memcpy((char*)v_cache + slot * row_bytes, (const char*)v + r * row_bytes, row_bytes);
    }
  return PKVO_OK;
}

/*
 * Varlen attention whose keys come from the paged cache: query rows
 * cu_q[b] .. cu_q[b+1]-1 of request b attend the first seqlens_k[b] tokens
 * of sequence b, read through its block-table row, no mask.  This is the
 * "Jalur Varlen" computation with the key rows found by the "Jalur decode"
 * address rule; each (row, head) is the three-step recipe of inference-notes
 * section 2, exactly as for a decode query.
 *
 *   q            [total_q, Hq, D] dtype
 *   k_cache, v_cache [num_blocks, bs, Hkv, D]
 *   block_table  [batch, max_blocks_per_seq] int32
 *   cu_q [batch+1], seqlens_k [batch] int32
 *   rows         q rows whose output is wanted (NULL = all)
 *   out          [n_eval, Hq, D] fp64
 */
int pkvo_varlen_paged(int dtype, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* cu_q, const int32_t* seqlens_k,
                      int max_len_q, int max_len_k, int batch, int total_q, int Hq, int Hkv,
                      int D, int num_blocks, int bs, int max_blocks_per_seq, double scale,
                      const int32_t* rows, int n_rows, double* out, int n_threads) {
  if (batch < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || Hq % Hkv != 0 || (dtype != PKVO_F32 && dtype != PKVO_BF16))
    return PKVO_ERR_ARGS;
  if (cu_q[0] != 0 || cu_q[batch] != total_q) return PKVO_ERR_CU;
  for (int b = 0; b < batch; ++b) {
    const int lq = cu_q[b + 1] - cu_q[b], lk = seqlens_k[b];
    if (lq < 0) return PKVO_ERR_CU;
    if (lk < 0) return PKVO_ERR_SEQLEN;
    if (lq > max_len_q || lk > max_len_k) return PKVO_ERR_MAXLEN;
    const int nblk = (lk + bs - 1) / bs;
    if (nblk > max_blocks_per_seq) return PKVO_ERR_TABLE_SPAN;
    for (int j = 0; j < nblk; ++j) {
      const int32_t pb = block_table[(int64_t)b * max_blocks_per_seq + j];
      if (pb < 0 || pb >= num_blocks) return PKVO_ERR_BLOCK;
    }
  }
  const int n_eval = rows ? n_rows : total_q;
  for (int e = 0; e < n_eval; ++e)
    if (rows && (rows[e] < 0 || rows[e] >= total_q)) return PKVO_ERR_ARGS;
  int32_t* req = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total_q > 0 ? total_q : 1));
  int rc = pkvo_request_index(cu_q, batch, total_q, req);
  if (rc) {
    free(req);
    return rc;
  }
  const int G = Hq / Hkv;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
  const int64_t units = (int64_t)n_eval * Hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_len_k > 0 ? max_len_k : 1));
#pragma omp for schedule(dynamic, 4)
    for (int64_t uidx = 0; uidx < units; ++uidx) {
      const int e = (int)(uidx / Hq), h = (int)(uidx % Hq);
      const int r = rows ? rows[e] : e;
      const int b = req[r];
      /* q row r is addressed as "sequence" r of a [total_q, 1, Hq, D] batch */
      decode_one(dtype, q, k_cache, v_cache, block_table + (int64_t)b * max_blocks_per_seq,
                 seqlens_k[b], r, h, G, Hq, Hkv, D, bs, scale, s,
                 out + ((int64_t)e * Hq + h) * D);
    }
    free(s);
  }
  free(req);
  return PKVO_OK;
}

/* Number of threads OpenMP would use (reported beside CPU timings). */
int pkvo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
