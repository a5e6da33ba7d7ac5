/*
 * pa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct fp64 CPU statement of causal grouped-query
 * attention over a paged KV cache.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it.  It shares no code, header, table or
 * helper with the GPU library and includes none of its files.
 *
 * What is computed (sources: the XY-Serve verdict page, "key_machinery" -- one
 * attention primitive is the matmul-softmax-matmul pattern over a tile of
 * queries and a K/V length; "core_discovery" -- K/V live in a PagedAttention-
 * style block cache, and prefill, decode and verify tokens are batched
 * together; the review "Understanding Inference Scaling for LLMs", Reference
 * graph entry [4], names grouped-query attention, where a group of query heads
 * shares one K/V head):
 *
 *   for every sequence s with n_s keys and q_s = qsl[s+1]-qsl[s] queries,
 *   every window row i < q_s (query token r = qsl[s]+i, absolute position
 *   p = n_s - q_s + i, bottom-right causal alignment) and every query head h
 *   (K/V head g = h / (Hq/Hkv)):
 *       x_j   = scale * sum_d q[r][h][d] * K_s[j][g][d]      for keys j = 0..p
 *       m     = max_j x_j,  w_j = exp(x_j - m),  l = sum_j w_j
 *       out[r][h][d] = sum_j w_j * V_s[j][g][d] / l
 *       lse[r][h]    = m + ln(l)                  (natural log of the scaled scores)
 *   where logical key j of sequence s lives in physical page
 *   pg = block_table[s][j / 16], slot t = j % 16, and
 *       K_s[j][g][d] = k_pool[pg][g][t][d]        (k_pool is [NP][Hkv][16][D])
 *       V_s[j][g][d] = v_pool[pg][g][d][t]        (v_pool is [NP][Hkv][D][16])
 *
 * Every element is widened to double exactly (bf16 bits << 16 is an exact
 * float); the whole computation is in double, two passes, no online softmax,
 * no key splitting.  Rows are independent; OpenMP runs them in parallel
 * without changing any arithmetic order.
 *
 * Also here: the page walk that gathers one sequence's K or V rows into a
 * dense array (bit copy) and the log-sum-exp merge of attention results over
 * disjoint key sets:
 *       lse = ln sum_i exp(lse_i),   o = sum_i exp(lse_i - lse) * o_i
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PAGE 16

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_BAD_CONTENT = 2, ORACLE_NO_MEMORY = 3 };

static double widen(const void* base, int dtype, int64_t idx) {
  if (dtype == ORACLE_BF16) {
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

/* Element offsets of (page, kv head, slot, d) in the two pool layouts. */
static int64_t k_offset(int64_t pg, int g, int t, int d, int Hkv, int D) {
  return ((pg * Hkv + g) * ORACLE_PAGE + t) * (int64_t)D + d;
}
static int64_t v_offset(int64_t pg, int g, int t, int d, int Hkv, int D) {
  return ((pg * Hkv + g) * (int64_t)D + d) * ORACLE_PAGE + t;
}

int oracle_abi_version(void) { return 1; }

/* Check that the batch description is self-consistent; returns ORACLE_OK or an error. */
static int check_batch(int B, int Hq, int Hkv, int D, int num_pages, int max_pages,
                       const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || num_pages < 0 || max_pages < 0)
    return ORACLE_BAD_ARG;
  if (B > 0 && qsl[0] != 0) return ORACLE_BAD_CONTENT;
  for (int s = 0; s < B; ++s) {
    int n = seq_lens[s], q = qsl[s + 1] - qsl[s];
    if (n < 0 || q < 0 || q > n) return ORACLE_BAD_CONTENT;
    int pages = (n + ORACLE_PAGE - 1) / ORACLE_PAGE;
    if (pages > max_pages) return ORACLE_BAD_CONTENT;
    for (int j = 0; j < pages; ++j) {
      int pg = block_table[(int64_t)s * max_pages + j];
      if (pg < 0 || pg >= num_pages) return ORACLE_BAD_CONTENT;
    }
  }
  return ORACLE_OK;
}

/*
 * out: double [T_q][Hq][D], lse: double [T_q][Hq]; T_q = qsl[B].
 * nthreads <= 0 lets OpenMP choose.  Returns ORACLE_OK or an error code.
 */
int oracle_attention(int B, int Hq, int Hkv, int D, int dtype, int num_pages, int max_pages,
                     const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl,
                     double scale, double* out, double* lse, int nthreads) {
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_BAD_ARG;
  int rc = check_batch(B, Hq, Hkv, D, num_pages, max_pages, block_table, seq_lens, qsl);
  if (rc != ORACLE_OK) return rc;
  const int G = Hq / Hkv;
  const int64_t T = B > 0 ? qsl[B] : 0;
  int max_n = 0;
  for (int s = 0; s < B; ++s) max_n = seq_lens[s] > max_n ? seq_lens[s] : max_n;

  /* row -> sequence map, so one flat parallel loop covers all (row, head) pairs */
  int32_t* row_seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  if (!row_seq) return ORACLE_NO_MEMORY;
  for (int s = 0; s < B; ++s)
    for (int32_t r = qsl[s]; r < qsl[s + 1]; ++r) row_seq[r] = s;

  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(max_n > 0 ? max_n : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!x || !acc) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t rh = 0; rh < T * Hq; ++rh) {
      if (!x || !acc) continue;
      const int64_t r = rh / Hq;
      const int h = (int)(rh % Hq);
      const int s = row_seq[r];
      const int g = h / G;
      const int n = seq_lens[s];
      const int qn = qsl[s + 1] - qsl[s];
      const int i = (int)(r - qsl[s]);
      const int p = n - qn + i; /* last visible key */
      const int32_t* bt = block_table + (int64_t)s * max_pages;
      const int64_t qoff = (r * Hq + h) * (int64_t)D;

      /* pass 1: scores and their maximum */
      double m = -INFINITY;
      for (int j = 0; j <= p; ++j) {
        const int64_t pg = bt[j / ORACLE_PAGE];
        const int t = j % ORACLE_PAGE;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += widen(q, dtype, qoff + d) * widen(k_pool, dtype, k_offset(pg, g, t, d, Hkv, D));
        x[j] = scale * dot;
        if (x[j] > m) m = x[j];
      }
      /* pass 2: weights, their sum and the weighted V rows */
      double l = 0.0;
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      for (int j = 0; j <= p; ++j) {
        const int64_t pg = bt[j / ORACLE_PAGE];
        const int t = j % ORACLE_PAGE;
        const double w = exp(x[j] - m);
        l += w;
        for (int d = 0; d < D; ++d) acc[d] += w * widen(v_pool, dtype, v_offset(pg, g, t, d, Hkv, D));
      }
      for (int d = 0; d < D; ++d) out[qoff + d] = acc[d] / l;
      lse[r * Hq + h] = m + log(l);
    }
    free(x);
    free(acc);
  }
  free(row_seq);
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Tree-structured verify windows (XY-Serve verdict page, referee_report
 * "significance" and desk_editor letter: verification of speculative token
 * trees).  Row i of a window of q <= 64 tokens over n keys sees every context
 * key j < n - q, and window key j = n - q + k only where bit k of
 * tree_mask[r] is set, and never a key past its own position n - q + i.  Rows
 * of windows longer than 64 follow the causal rule (their mask is ignored).
 * A row that sees no key gets out = 0 and lse = -inf.  Otherwise the same
 * two-pass fp64 computation as oracle_attention.
 */
static int tree_visible(int j, int p, int win0, int qn, uint64_t mask) {
  if (j > p) return 0;
  if (j < win0 || qn > 64) return 1;
  return (int)((mask >> (j - win0)) & 1u);
}

int oracle_attention_tree(int B, int Hq, int Hkv, int D, int dtype, int num_pages, int max_pages,
                          const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl,
                          const uint64_t* tree_mask, double scale, double* out, double* lse) {
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_BAD_ARG;
  int rc = check_batch(B, Hq, Hkv, D, num_pages, max_pages, block_table, seq_lens, qsl);
  if (rc != ORACLE_OK) return rc;
  const int G = Hq / Hkv;
  int max_n = 0;
  for (int s = 0; s < B; ++s) max_n = seq_lens[s] > max_n ? seq_lens[s] : max_n;
  double* x = (double*)malloc(sizeof(double) * (size_t)(max_n > 0 ? max_n : 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)D);
  if (!x || !acc) {
    free(x);
    free(acc);
    return ORACLE_NO_MEMORY;
  }
  for (int s = 0; s < B; ++s) {
    const int n = seq_lens[s];
    const int qn = qsl[s + 1] - qsl[s];
    const int win0 = n - qn;
    const int32_t* bt = block_table + (int64_t)s * max_pages;
    for (int i = 0; i < qn; ++i) {
      const int64_t r = qsl[s] + i;
      const int p = win0 + i;
      for (int h = 0; h < Hq; ++h) {
        const int kvh = h / G; /* K/V head read by query head h */
        const int64_t qrow = (r * Hq + h) * (int64_t)D;
        double m = -INFINITY;
        for (int j = 0; j <= p; ++j) {
          if (!tree_visible(j, p, win0, qn, tree_mask[r])) continue;
          const int64_t page = bt[j / ORACLE_PAGE];
          const int slot = j % ORACLE_PAGE;
          double qk = 0.0;
          for (int d = 0; d < D; ++d)
            qk += widen(q, dtype, qrow + d) * widen(k_pool, dtype, k_offset(page, kvh, slot, d, Hkv, D));
          x[j] = qk * scale;
          m = x[j] > m ? x[j] : m;
        }
        double l = 0.0;
        for (int d = 0; d < D; ++d) acc[d] = 0.0;
        for (int j = 0; j <= p; ++j) {
          if (!tree_visible(j, p, win0, qn, tree_mask[r])) continue;
          const int64_t page = bt[j / ORACLE_PAGE];
          const int slot = j % ORACLE_PAGE;
          const double wj = exp(x[j] - m);
          l += wj;
          for (int d = 0; d < D; ++d) acc[d] += wj * widen(v_pool, dtype, v_offset(page, kvh, slot, d, Hkv, D));
        }
        for (int d = 0; d < D; ++d) out[qrow + d] = l > 0.0 ? acc[d] / l : 0.0;
        lse[r * Hq + h] = l > 0.0 ? m + log(l) : -INFINITY;
      }
    }
  }
  free(x);
  free(acc);
  return ORACLE_OK;
}

/*
 * FP8 KV pages (the Arctic review lists quantized KV caches among the
 * serving optimizations; OCP FP8 E4M3 is the MI355X's native 8-bit float).
 * A code is decoded from the E4M3 definition: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); the code
 * with all exponent and mantissa bits set is NaN; there is no infinity.
 */
double oracle_fp8_decode(int code) {
  const int sgn = (code >> 7) & 1, ex = (code >> 3) & 15, man = code & 7;
  if (ex == 15 && man == 7) return NAN;
  const double mag = ex == 0 ? ldexp(man / 8.0, -6) : ldexp(1.0 + man / 8.0, ex - 7);
  return sgn ? -mag : mag;
}

/*
 * Attention over FP8 pages: q is bf16; k_codes / v_codes hold E4M3 codes in
 * the pool layouts above; k_scale / v_scale [NP][Hkv] fp32 hold one scale per
 * (page, kv head).  Key j of sequence s is k = decode(code) * k_scale[pg][g],
 * and V likewise; then exactly the computation of oracle_attention.
 */
int oracle_attention_fp8(int B, int Hq, int Hkv, int D, int num_pages, int max_pages, const uint16_t* q,
                         const uint8_t* k_codes, const uint8_t* v_codes, const float* k_scale, const float* v_scale,
                         const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl, double scale,
                         double* out, double* lse, int nthreads) {
  int rc = check_batch(B, Hq, Hkv, D, num_pages, max_pages, block_table, seq_lens, qsl);
  if (rc != ORACLE_OK) return rc;
  const int G = Hq / Hkv;
  const int64_t T = B > 0 ? qsl[B] : 0;
  int max_n = 0;
  for (int s = 0; s < B; ++s) max_n = seq_lens[s] > max_n ? seq_lens[s] : max_n;
  double table[256];
  for (int c = 0; c < 256; ++c) table[c] = oracle_fp8_decode(c);
  int32_t* row_seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  if (!row_seq) return ORACLE_NO_MEMORY;
  for (int s = 0; s < B; ++s)
    for (int32_t r = qsl[s]; r < qsl[s + 1]; ++r) row_seq[r] = s;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)(max_n > 0 ? max_n : 1));
    double* num = (double*)malloc(sizeof(double) * (size_t)D);
    if (!sc || !num) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t rh = 0; rh < T * Hq; ++rh) {
      if (!sc || !num) continue;
      const int64_t r = rh / Hq;
      const int h = (int)(rh % Hq);
      const int s = row_seq[r];
      const int kvh = h / G;
      const int n = seq_lens[s];
      const int last = n - (qsl[s + 1] - qsl[s]) + (int)(r - qsl[s]);
      const int32_t* bt = block_table + (int64_t)s * max_pages;
      const int64_t qrow = (r * Hq + h) * (int64_t)D;
      double mx = -INFINITY;
      for (int j = 0; j <= last; ++j) {
        const int64_t page = bt[j / ORACLE_PAGE];
        const int slot = j % ORACLE_PAGE;
        const double ks = (double)k_scale[page * Hkv + kvh];
        double qk = 0.0;
        for (int d = 0; d < D; ++d)
          qk += widen(q, ORACLE_BF16, qrow + d) * (table[k_codes[k_offset(page, kvh, slot, d, Hkv, D)]] * ks);
        sc[j] = qk * scale;
        mx = sc[j] > mx ? sc[j] : mx;
      }
      double den = 0.0;
      for (int d = 0; d < D; ++d) num[d] = 0.0;
      for (int j = 0; j <= last; ++j) {
        const int64_t page = bt[j / ORACLE_PAGE];
        const int slot = j % ORACLE_PAGE;
        const double vs = (double)v_scale[page * Hkv + kvh];
        const double wj = exp(sc[j] - mx);
        den += wj;
        for (int d = 0; d < D; ++d) num[d] += wj * (table[v_codes[v_offset(page, kvh, slot, d, Hkv, D)]] * vs);
      }
      for (int d = 0; d < D; ++d) out[qrow + d] = num[d] / den;
      lse[r * Hq + h] = mx + log(den);
    }
    free(sc);
    free(num);
  }
  free(row_seq);
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Gather sequence `seq`'s rows of one pool into dense [Hkv][n][D] order by
 * walking its block table (element bytes copied unchanged).
 * which = 0: K pool layout [NP][Hkv][16][D]; which = 1: V pool layout [NP][Hkv][D][16].
 */
int oracle_gather(int which, int dtype, int Hkv, int D, int num_pages, int max_pages, const void* pool,
                  const int32_t* block_table, const int32_t* seq_lens, int seq, void* dense) {
  if ((which != 0 && which != 1) || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return ORACLE_BAD_ARG;
  const int n = seq_lens[seq];
  const size_t eb = dtype == ORACLE_BF16 ? 2 : 4;
  const int32_t* bt = block_table + (int64_t)seq * max_pages;
  for (int j = 0; j < n; ++j) {
    const int64_t pg = bt[j / ORACLE_PAGE];
    if (pg < 0 || pg >= num_pages) return ORACLE_BAD_CONTENT;
  }
  for (int g = 0; g < Hkv; ++g)
    for (int j = 0; j < n; ++j) {
      const int64_t pg = bt[j / ORACLE_PAGE];
      const int t = j % ORACLE_PAGE;
      for (int d = 0; d < D; ++d) {
        const int64_t src = which == 0 ? k_offset(pg, g, t, d, Hkv, D) : v_offset(pg, g, t, d, Hkv, D);
        const int64_t dst = ((int64_t)g * n + j) * D + d;
        memcpy((char*)dense + dst * eb, (const char*)pool + src * eb, eb);
      }
    }
  return ORACLE_OK;
}

/*
 * Paged KV append: the K/V rows of a batch's new tokens go into their pages.
 * New token i of sequence s (query token r = qsl[s] + i) sits at position
 * p = n_s - q_s + i -- the same reading as the attention above, where seq_lens
 * count the new tokens -- so, with pg = block_table[s][p / 16], t = p % 16:
 *     k_pool[pg][g][t][d] = k_new[r][g][d],   v_pool[pg][g][d][t] = v_new[r][g][d]
 * for every K/V head g and d (element bits copied).  k_new and v_new are
 * [T_q][Hkv][D].  Nothing else in the pools changes.  (XY-Serve verdict page,
 * "core_discovery": K/V live in a PagedAttention-style block cache that every
 * step appends to.)
 */
int oracle_append(int B, int Hkv, int D, int dtype, int num_pages, int max_pages, const int32_t* block_table,
                  const int32_t* seq_lens, const int32_t* qsl, const void* k_new, const void* v_new, void* k_pool,
                  void* v_pool) {
  if (B < 0 || Hkv <= 0 || D <= 0 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return ORACLE_BAD_ARG;
  const size_t eb = dtype == ORACLE_BF16 ? 2 : 4;
  if (B > 0 && qsl[0] != 0) return ORACLE_BAD_CONTENT;
  for (int s = 0; s < B; ++s) {
    const int n = seq_lens[s], q = qsl[s + 1] - qsl[s];
    if (q < 0 || q > n || (n + ORACLE_PAGE - 1) / ORACLE_PAGE > max_pages) return ORACLE_BAD_CONTENT;
    for (int p = n - q; p < n; ++p) {
      const int64_t pg = block_table[(int64_t)s * max_pages + p / ORACLE_PAGE];
      if (pg < 0 || pg >= num_pages) return ORACLE_BAD_CONTENT;
    }
  }
  for (int s = 0; s < B; ++s) {
    const int n = seq_lens[s], q = qsl[s + 1] - qsl[s];
    for (int i = 0; i < q; ++i) {
      const int64_t r = qsl[s] + i;
      const int p = n - q + i;
      const int64_t pg = block_table[(int64_t)s * max_pages + p / ORACLE_PAGE];
      const int t = p % ORACLE_PAGE;
      for (int g = 0; g < Hkv; ++g)
        for (int d = 0; d < D; ++d) {
          const int64_t src = (r * Hkv + g) * D + d;
          memcpy((char*)k_pool + k_offset(pg, g, t, d, Hkv, D) * eb, (const char*)k_new + src * eb, eb);
          memcpy((char*)v_pool + v_offset(pg, g, t, d, Hkv, D) * eb, (const char*)v_new + src * eb, eb);
        }
    }
  }
  return ORACLE_OK;
}

/*
 * Combine attention results computed over disjoint key sets.
 * o_parts: [P][rows][D], lse_parts: [P][rows]  ->  o: [rows][D], lse: [rows].
 * A part with lse = -inf (it saw no key) contributes nothing.
 */
int oracle_merge(int P, int64_t rows, int D, const double* o_parts, const double* lse_parts,
                 double* o, double* lse) {
  if (P <= 0 || rows < 0 || D <= 0) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < rows; ++r) {
    double m = -INFINITY;
    for (int i = 0; i < P; ++i)
      if (lse_parts[(int64_t)i * rows + r] > m) m = lse_parts[(int64_t)i * rows + r];
    double sum = 0.0;
    for (int i = 0; i < P; ++i) sum += exp(lse_parts[(int64_t)i * rows + r] - m);
    const double total = m + log(sum);
    for (int d = 0; d < D; ++d) {
      double v = 0.0;
      for (int i = 0; i < P; ++i) {
        const double li = lse_parts[(int64_t)i * rows + r];
        if (li == -INFINITY) continue;
        v += exp(li - total) * o_parts[((int64_t)i * rows + r) * D + d];
      }
      o[r * D + d] = v;
    }
    lse[r] = total;
  }
  return ORACLE_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
