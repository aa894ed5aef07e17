/*
 * swa_oracle.c -- plain, slow, obviously-correct CPU reference for
 * sliding-window grouped-query attention.  TEST INFRASTRUCTURE ONLY: the
 * tests, the smoke check and the CPU-baseline leg of the benchmark call it;
 * the GPU library never links or calls it, and it shares no code with it.
 *
 * Everything is computed in IEEE double.  bf16 inputs are widened exactly
 * (a bf16 bit pattern is the upper half of an fp32 bit pattern) and fp32
 * inputs are widened exactly; there is no blocking, no fusion and no online
 * rescaling: every output row scans its allowed keys twice (max, then sum).
 *
 * Pages cited (title; section):
 *   [SPYRE]  "Enable compact sliding-window attention for Gemma 3 and Gemma 4
 *            variants" (torch-spyre/hf-adapters pull request 496)
 *   [BONSAI] "Gemma3 Local Attention Cache" (jax-ml/bonsai issue 124)
 *   [SDPA]   "Add SDPA attention implementation" (ServiceNow/Fast-LLM pull
 *            request 512)
 *
 * Readings where the pages are silent:
 *   - window W keeps key j for query i iff 0 <= i - j < W (W keys, self
 *     included); W <= 0 means no window (a global layer);
 *   - the window is one-sided: keys after the query (allowed only inside an
 *     image block) never fail the window term;
 *   - an image block is a maximal run of consecutive tokens of one document
 *     carrying the same non-negative id; id -1 marks a text token;
 *   - a query with no allowed key yields a zero row;
 *   - query head h reads key/value head h / (Hq / Hkv).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_F32 1

#define ORACLE_CAUSAL 0
#define ORACLE_BLOCKWISE 1

/* Exact widening of element `idx` of a bf16 or fp32 array to double. */
static double load_elem(const void* base, int dtype, size_t idx) {
  if (dtype == ORACLE_BF16) {
    uint16_t h = ((const uint16_t*)base)[idx];
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

/* Index of the document holding packed token t: the d with
 * cu[d] <= t < cu[d+1].  Documents come from cu_seqlens, the packing input
 * named in [SDPA] Summary.  Linear scan: the oracle favours obviousness. */
static int doc_of(const int32_t* cu, int ndocs, int t) {
  for (int d = 0; d < ndocs; ++d)
    if (t >= cu[d] && t < cu[d + 1]) return d;
  return -1;
}

/* Same image block: both tokens carry the same non-negative id and every
 * token between them carries it too (a maximal run inside one document).
 * [SPYRE] Summary: the sliding mask admits the vision-blockwise pairs. */
static int same_block(const int32_t* ids, int i, int j) {
  if (ids[i] < 0 || ids[j] != ids[i]) return 0;
  int a = i < j ? i : j, b = i < j ? j : i;
  for (int t = a; t <= b; ++t)
    if (ids[t] != ids[i]) return 0;
  return 1;
}

/* The mask for query i and key j of one document.
 * [SPYRE] Summary: sliding layers use window AND (causal OR vision-blockwise);
 * global (unwindowed) layers are causal.  [SDPA] Summary: keys outside the
 * query's document are excluded. */
int oracle_allowed(const int32_t* cu, int ndocs, const int32_t* ids, int window,
                   int mode, int i, int j) {
  int di = doc_of(cu, ndocs, i), dj = doc_of(cu, ndocs, j);
  if (di < 0 || di != dj) return 0;
  int in_window = (window <= 0) || (i - j < window);
  int causal = (j <= i);
  int blockwise = (mode == ORACLE_BLOCKWISE) && ids != NULL && same_block(ids, i, j);
  return in_window && (causal || blockwise);
}

/* One output row: out[0..d) = sum_j softmax(scale * <q, k_j>) v_j over the
 * keys listed in `keys` (already filtered by the mask), in double.  Query
 * row, key rows and value rows are addressed by element offsets.  When
 * `lse` is given it receives log(sum_j exp(scale * <q, k_j>)), the row's
 * log-sum-exp (-inf for an empty set). */
static void attend_row(const void* q, size_t q_off, const void* k, const void* v,
                       const size_t* kv_offs, int nkeys, int dtype, int d,
                       double scale, double* s_buf, double* out, double* lse) {
  for (int e = 0; e < d; ++e) out[e] = 0.0;
  if (lse) *lse = -INFINITY;
  if (nkeys == 0) return; /* empty allowed set: zero row */
  double m = -INFINITY;
  for (int t = 0; t < nkeys; ++t) {
    double dot = 0.0;
    for (int e = 0; e < d; ++e)
      dot += load_elem(q, dtype, q_off + e) * load_elem(k, dtype, kv_offs[t] + e);
    s_buf[t] = scale * dot;
    if (s_buf[t] > m) m = s_buf[t];
  }
  double l = 0.0;
  for (int t = 0; t < nkeys; ++t) {
    double p = exp(s_buf[t] - m);
    l += p;
    for (int e = 0; e < d; ++e) out[e] += p * load_elem(v, dtype, kv_offs[t] + e);
  }
  for (int e = 0; e < d; ++e) out[e] /= l;
  if (lse) *lse = m + log(l);
}

/*
 * Packed variable-length prefill.
 *   q   [T, hq, d], k and v [T, hkv, d]  (bf16 bit patterns or fp32)
 *   cu  int32[ndocs + 1], cu[0] = 0, cu[ndocs] = T, non-decreasing
 *   ids int32[T] image-block ids (-1 = text); read only when mode = BLOCKWISE
 *   rows: the packed query indices to compute (NULL = all T rows, nrows = T)
 *   out double[nrows, hq, d]
 *   lse double[nrows, hq] or NULL: each row's log-sum-exp of its scaled scores
 * Returns 0, or -1 on malformed arguments.
 */
int oracle_prefill_rows(const void* q, const void* k, const void* v, int dtype,
                        const int32_t* cu, int ndocs, const int32_t* ids,
                        int window, int mode, int T, int hq, int hkv, int d,
                        double scale, const int32_t* rows, int nrows,
                        double* out, double* lse, int nthreads) {
  if (hkv <= 0 || hq % hkv != 0 || d <= 0 || ndocs < 0 || T < 0) return -1;
  if (cu[0] != 0 || cu[ndocs] != T) return -1;
  for (int dd = 0; dd < ndocs; ++dd)
    if (cu[dd + 1] < cu[dd]) return -1;
  if (mode == ORACLE_BLOCKWISE && ids == NULL && T > 0) return -1;
  const int g = hq / hkv; /* [SDPA] Summary: K/V are repeated per query head */
  int n = rows ? nrows : T;
  long long total = (long long)n * hq;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int err = 0;
#pragma omp parallel
  {
    size_t* offs = (size_t*)malloc(sizeof(size_t) * (size_t)(T > 0 ? T : 1));
    double* sbuf = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    if (!offs || !sbuf) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (long long w = 0; w < total; ++w) {
      if (!offs || !sbuf) continue;
      int r = (int)(w / hq), h = (int)(w % hq);
      int i = rows ? rows[r] : r;
      double* o = out + ((size_t)r * hq + h) * d;
      if (i < 0 || i >= T) {
        for (int e = 0; e < d; ++e) o[e] = NAN;
        if (lse) lse[(size_t)r * hq + h] = NAN;
        continue;
      }
      int kvh = h / g;
      int di = doc_of(cu, ndocs, i);
      int nk = 0;
      for (int j = cu[di]; j < cu[di + 1]; ++j)
        if (oracle_allowed(cu, ndocs, ids, window, mode, i, j))
          offs[nk++] = ((size_t)j * hkv + kvh) * d;
      attend_row(q, ((size_t)i * hq + h) * d, k, v, offs, nk, dtype, d, scale,
                 sbuf, o, lse ? lse + (size_t)r * hq + h : NULL);
    }
    free(offs);
    free(sbuf);
  }
  return err ? -1 : 0;
}

/*
 * One-token decode against a LINEAR (never wrapped) history of each
 * sequence.  Sequence b stores positions [first_pos[b], first_pos[b] +
 * hist_len[b]) at rows hist_off[b] .. of k_lin / v_lin [rows, hkv, d].
 * The query of sequence b sits at position pos[b]; positions below lo[b]
 * are left padding and never attended ([SPYRE] Summary keeps left padding).
 * The allowed keys are max(lo, pos - W + 1, 0) <= a <= pos.
 *   q double-able [B, hq, d]; out double[B, hq, d].
 * Returns 0, -1 on malformed arguments, -2 when a history does not cover
 * the allowed positions.
 */
int oracle_decode_linear(const void* q, const void* k_lin, const void* v_lin,
                         int dtype, const int64_t* hist_off,
                         const int32_t* first_pos, const int32_t* hist_len,
                         const int32_t* pos, const int32_t* lo, int window,
                         int B, int hq, int hkv, int d, double scale,
                         double* out, int nthreads) {
  if (hkv <= 0 || hq % hkv != 0 || d <= 0 || B < 0) return -1;
  const int g = hq / hkv;
  for (int b = 0; b < B; ++b) {
    int lower = lo[b] > 0 ? lo[b] : 0;
    if (window > 0 && pos[b] - window + 1 > lower) lower = pos[b] - window + 1;
    if (pos[b] < 0) return -1;
    if (lower <= pos[b] &&
        (first_pos[b] > lower || first_pos[b] + hist_len[b] <= pos[b]))
      return -2;
  }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int maxw = 1;
  for (int b = 0; b < B; ++b)
    if (hist_len[b] > maxw) maxw = hist_len[b];
  int err = 0;
#pragma omp parallel
  {
    size_t* offs = (size_t*)malloc(sizeof(size_t) * (size_t)maxw);
    double* sbuf = (double*)malloc(sizeof(double) * (size_t)maxw);
    if (!offs || !sbuf) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (long long w = 0; w < (long long)B * hq; ++w) {
      if (!offs || !sbuf) continue;
      int b = (int)(w / hq), h = (int)(w % hq), kvh = h / g;
      int lower = lo[b] > 0 ? lo[b] : 0;
      if (window > 0 && pos[b] - window + 1 > lower) lower = pos[b] - window + 1;
      int nk = 0;
      for (int a = lower; a <= pos[b]; ++a) {
        size_t row = (size_t)hist_off[b] + (size_t)(a - first_pos[b]);
        offs[nk++] = (row * hkv + kvh) * d;
      }
      attend_row(q, ((size_t)b * hq + h) * d, k_lin, v_lin, offs, nk, dtype, d,
                 scale, sbuf, out + ((size_t)b * hq + h) * d, NULL);
    }
    free(offs);
    free(sbuf);
  }
  return err ? -1 : 0;
}

/* Gradient quantities of one query row (packed index i, query head h) of
 * the prefill, in double, for the loss whose gradient with respect to the
 * row's output is dO (dout[i, h]).  The forward is recomputed from its
 * definition: the allowed keys j (listed in `keys`), the softmax weights
 * p_j of the row's scores scale * <q_i, k_j>, and dp_j = <dO, v_j> (the
 * gradient with respect to p_j, since the output is sum_j p_j v_j).
 * `*delta` = sum_j p_j dp_j, the term the softmax's Jacobian subtracts:
 * the gradient with respect to the score j is p_j (dp_j - delta).
 * Returns the number of allowed keys. */
static int row_grad_terms(const void* q, const void* k, const void* v, const void* dout,
                          int dtype, const int32_t* cu, int ndocs, const int32_t* ids,
                          int window, int mode, int hq, int hkv, int d, double scale,
                          int i, int h, int* keys, double* p, double* dp, double* delta) {
  const int g = hq / hkv, kvh = h / g;
  const int di = doc_of(cu, ndocs, i);
  *delta = 0.0;
  if (di < 0) return 0;
  const size_t qo = ((size_t)i * hq + h) * d;
  int nk = 0;
  double m = -INFINITY;
  for (int j = cu[di]; j < cu[di + 1]; ++j) {
    if (!oracle_allowed(cu, ndocs, ids, window, mode, i, j)) continue;
    const size_t ko = ((size_t)j * hkv + kvh) * d;
    double dot = 0.0, dov = 0.0;
    for (int e = 0; e < d; ++e) {
      dot += load_elem(q, dtype, qo + e) * load_elem(k, dtype, ko + e);
      dov += load_elem(dout, dtype, qo + e) * load_elem(v, dtype, ko + e);
    }
    keys[nk] = j;
    p[nk] = scale * dot;
    dp[nk] = dov;
    if (p[nk] > m) m = p[nk];
    ++nk;
  }
  double l = 0.0;
  for (int t = 0; t < nk; ++t) {
    p[t] = exp(p[t] - m);
    l += p[t];
  }
  double dl = 0.0;
  for (int t = 0; t < nk; ++t) {
    p[t] /= l;
    dl += p[t] * dp[t];
  }
  *delta = dl;
  return nk;
}

/*
 * Backward of the packed variable-length prefill: the gradients of the
 * loss L = sum over rows and heads of <dout[i, h], out[i, h]> with respect
 * to q, k and v, in double, by the chain rule through the definition
 * (out = sum_j p_j v_j, p = softmax of the scores, score_j = scale <q, k_j>):
 *   dv[j, kvh] = sum over rows i and heads h of the group: p_ij dout[i, h]
 *   ds_ij      = p_ij (dp_ij - delta_i)
 *   dq[i, h]   = scale * sum_j ds_ij k[j, kvh]
 *   dk[j, kvh] = scale * sum over rows i and heads h of the group: ds_ij q[i, h]
 * (the GQA head map sends every query head of a group to the same K/V head,
 * so their contributions add up).
 *   rows: packed query rows whose dq to compute (NULL = all T), dq double[nrows, hq, d]
 *   keys: packed key rows whose dk, dv to compute (NULL = all T), dk and dv
 *         double[nkeys, hkv, d]
 * Returns 0, or -1 on malformed arguments.
 */
int oracle_prefill_backward(const void* q, const void* k, const void* v, const void* dout,
                            int dtype, const int32_t* cu, int ndocs, const int32_t* ids,
                            int window, int mode, int T, int hq, int hkv, int d,
                            double scale, const int32_t* rows, int nrows,
                            const int32_t* keys, int nkeys, double* dq, double* dk,
                            double* dv, int nthreads) {
  if (hkv <= 0 || hq % hkv != 0 || d <= 0 || ndocs < 0 || T < 0) return -1;
  if (cu[0] != 0 || cu[ndocs] != T) return -1;
  for (int dd = 0; dd < ndocs; ++dd)
    if (cu[dd + 1] < cu[dd]) return -1;
  if (mode == ORACLE_BLOCKWISE && ids == NULL && T > 0) return -1;
  const int g = hq / hkv;
  const int nr = rows ? nrows : T, nkr = keys ? nkeys : T;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int err = 0;
  const size_t cap = (size_t)(T > 0 ? T : 1);
#pragma omp parallel
  {
    int* kl = (int*)malloc(sizeof(int) * cap);
    double* p = (double*)malloc(sizeof(double) * cap);
    double* dp = (double*)malloc(sizeof(double) * cap);
    if (!kl || !p || !dp) {
#pragma omp atomic write
      err = 1;
    }
    /* dq: one (row, head) at a time */
#pragma omp for schedule(dynamic, 4)
    for (long long w = 0; w < (long long)nr * hq; ++w) {
      if (!kl || !p || !dp) continue;
      const int r = (int)(w / hq), h = (int)(w % hq), kvh = h / g;
      const int i = rows ? rows[r] : r;
      double* o = dq + ((size_t)r * hq + h) * d;
      for (int e = 0; e < d; ++e) o[e] = 0.0;
      if (i < 0 || i >= T) {
        for (int e = 0; e < d; ++e) o[e] = NAN;
        continue;
      }
      double delta;
      const int nk = row_grad_terms(q, k, v, dout, dtype, cu, ndocs, ids, window, mode, hq,
                                    hkv, d, scale, i, h, kl, p, dp, &delta);
      for (int t = 0; t < nk; ++t) {
        const double ds = p[t] * (dp[t] - delta);
        const size_t ko = ((size_t)kl[t] * hkv + kvh) * d;
        for (int e = 0; e < d; ++e) o[e] += scale * ds * load_elem(k, dtype, ko + e);
      }
    }
    /* dk, dv of every key: one K/V head per thread; each (row, head) of the
     * group adds its terms to the keys it admits */
#pragma omp for schedule(dynamic, 1)
    for (int kvh = 0; kvh < (keys ? 0 : hkv); ++kvh) {
      if (!kl || !p || !dp) continue;
      for (int j = 0; j < T; ++j)
        for (int e = 0; e < d; ++e)
          dk[((size_t)j * hkv + kvh) * d + e] = dv[((size_t)j * hkv + kvh) * d + e] = 0.0;
      for (int h = kvh * g; h < (kvh + 1) * g; ++h) {
        for (int i = 0; i < T; ++i) {
          double delta;
          const int nk = row_grad_terms(q, k, v, dout, dtype, cu, ndocs, ids, window, mode, hq,
                                        hkv, d, scale, i, h, kl, p, dp, &delta);
          const size_t qo = ((size_t)i * hq + h) * d;
          for (int t = 0; t < nk; ++t) {
            const double ds = p[t] * (dp[t] - delta);
            double* ok = dk + ((size_t)kl[t] * hkv + kvh) * d;
            double* ov = dv + ((size_t)kl[t] * hkv + kvh) * d;
            for (int e = 0; e < d; ++e) {
              ok[e] += scale * ds * load_elem(q, dtype, qo + e);
              ov[e] += p[t] * load_elem(dout, dtype, qo + e);
            }
          }
        }
      }
    }
    /* dk, dv of selected keys: one (key row, kv head) at a time, gathering
     * every (row, head) that admits the key */
#pragma omp for schedule(dynamic, 1)
    for (long long w = 0; w < (keys ? (long long)nkr * hkv : 0); ++w) {
      if (!kl || !p || !dp) continue;
      const int r = (int)(w / hkv), kvh = (int)(w % hkv);
      const int j = keys ? keys[r] : r;
      double* ok = dk + ((size_t)r * hkv + kvh) * d;
      double* ov = dv + ((size_t)r * hkv + kvh) * d;
      for (int e = 0; e < d; ++e) ok[e] = ov[e] = 0.0;
      if (j < 0 || j >= T) {
        for (int e = 0; e < d; ++e) ok[e] = ov[e] = NAN;
        continue;
      }
      const int dj = doc_of(cu, ndocs, j);
      if (dj < 0) continue;
      for (int i = cu[dj]; i < cu[dj + 1]; ++i) {
        if (!oracle_allowed(cu, ndocs, ids, window, mode, i, j)) continue;
        for (int h = kvh * g; h < (kvh + 1) * g; ++h) {
          double delta;
          const int nk = row_grad_terms(q, k, v, dout, dtype, cu, ndocs, ids, window, mode,
                                        hq, hkv, d, scale, i, h, kl, p, dp, &delta);
          int t = 0;
          while (t < nk && kl[t] != j) ++t;
          if (t == nk) continue; /* cannot happen: the mask admitted j */
          const double ds = p[t] * (dp[t] - delta);
          const size_t qo = ((size_t)i * hq + h) * d;
          for (int e = 0; e < d; ++e) {
            ok[e] += scale * ds * load_elem(q, dtype, qo + e);
            ov[e] += p[t] * load_elem(dout, dtype, qo + e);
          }
        }
      }
    }
    free(kl);
    free(p);
    free(dp);
  }
  return err ? -1 : 0;
}

/* Number of (query, key) pairs the mask admits over the whole packed batch,
 * counted one pair at a time.  Used to pin the mask against closed forms. */
long long oracle_count_allowed(const int32_t* cu, int ndocs, const int32_t* ids,
                               int window, int mode, int T, int nthreads) {
  long long total = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for reduction(+ : total) schedule(dynamic, 16)
  for (int i = 0; i < T; ++i) {
    int di = doc_of(cu, ndocs, i);
    for (int j = cu[di]; j < cu[di + 1]; ++j)
      total += oracle_allowed(cu, ndocs, ids, window, mode, i, j);
  }
  return total;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
