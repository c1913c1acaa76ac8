/*
 * oracle.c -- float64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check of the package entry
 * script and the CPU-baseline leg of the benchmark use it.  It shares no code,
 * header, table or helper with the HIP library; it is written from the
 * mathematics on the pages listed below and nothing else.
 *
 * Sources (web pages on FlashAttention; cited by title and section):
 *   [P1] "FlashAttention ontleed: snellere berekening via GPU-geheugen"
 *        (leren.llmnet.nl)
 *   [P3] "03. FlashAttention" (frontier-llm-systems notes)
 *   [P4] "FlashAttention" explainer (Lensa ML), Steps 1-6
 *
 * Everything is float64.  Layouts are row-major: a tensor of shape
 * [BH, N, d] is BH independent heads of N rows with d contiguous.
 * Inputs are the exact fp16/bf16 values the GPU receives, widened to double
 * by the caller, so input rounding is not counted as error.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes of the repository):
 *   - causal: key j is visible to query i iff j <= i (pages say "mask" only);
 *   - sliding window w > 0 (with causal): key j is visible to query i iff
 *     i - w < j <= i, the w most recent keys including the query's own
 *     position (the pages name the variant, not its formula);
 *   - grouped-query attention: H query heads share H_kv key/value heads in
 *     contiguous groups, query head h reading key/value head h / (H / H_kv)
 *     (the pages say several query heads share one key/value head);
 *   - lse: the natural-log log-sum-exp of the scaled, masked scores of a row,
 *     lse = m + ln(l);  a row with no visible key gets O = 0, lse = -inf;
 *   - scale multiplies Q K^T before masking and softmax (pages fix 1/sqrt(d));
 *   - backward: plain calculus of the three-step definition for a loss whose
 *     gradient with respect to O is dO.
 *
 * Parallelism: OpenMP over independent rows / columns only; every reduction
 * is a plain sequential loop, in definition order.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_ROWS_PER_TASK 32

/*
 * Visibility of key j from query i.  Causal masking [P4 Step 2 lists the mask
 * among the per-element operations]; the sliding window restricts the keys to
 * the window [P3 §"Variantes et extensions", sliding-window variant].
 */
static int oracle_visible(long i, long j, int causal, long window) {
  if (!causal) return 1;
  if (j > i) return 0;
  return window <= 0 || j > i - window;
}

static void oracle_set_threads(int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
}

/* Number of OpenMP threads a parallel region will use (for timing reports). */
int oracle_max_threads(void) { return omp_get_max_threads(); }

/*
 * Softmax of one row, by its definition: p_i = e^{x_i} / sum_j e^{x_j}
 * [P1 §"De wiskundige doorbraak: Tiling en Online Softmax", the softmax
 * formula], evaluated with the row maximum subtracted first so that no
 * exponent is positive [P3 §"Online softmax"; P4 Step 4, the fp16 overflow
 * remark].  Entries equal to -inf (masked) get probability 0.
 */
void oracle_softmax(const double* x, long n, double* p) {
  double m = -INFINITY;
  for (long i = 0; i < n; ++i) if (x[i] > m) m = x[i];
  if (m == -INFINITY) { for (long i = 0; i < n; ++i) p[i] = 0.0; return; }
  double s = 0.0;
  for (long i = 0; i < n; ++i) s += exp(x[i] - m);
  for (long i = 0; i < n; ++i) p[i] = exp(x[i] - m) / s;
}

/*
 * Online (one-pass) softmax over consecutive chunks of `chunk` scores
 * [P4 Step 4 "Online Softmax": running maximum m and running sum l; for each
 * chunk, m_new = max(m, chunk max) and l_new = l * e^{m - m_new} +
 * sum_{x in chunk} e^{x - m_new}; start m = -inf, l = 0].  After the last
 * chunk, p_i = e^{x_i - m} / l.  m_trace/l_trace (may be NULL) receive the
 * running (m, l) after each chunk.  Returns the number of chunks.
 */
long oracle_softmax_online(const double* x, long n, long chunk, double* p,
                           double* m_trace, double* l_trace) {
  double m = -INFINITY, l = 0.0;
  long nchunks = 0;
  for (long c0 = 0; c0 < n; c0 += chunk, ++nchunks) {
    long c1 = c0 + chunk < n ? c0 + chunk : n;
    double cmax = -INFINITY;
    for (long i = c0; i < c1; ++i) if (x[i] > cmax) cmax = x[i];
    double m_new = m > cmax ? m : cmax;
    if (m_new != -INFINITY) {
      double csum = 0.0;
      for (long i = c0; i < c1; ++i) csum += exp(x[i] - m_new);
      double rescale = (m == -INFINITY) ? 0.0 : exp(m - m_new);
      l = l * rescale + csum;
      m = m_new;
    }
    if (m_trace) m_trace[nchunks] = m;
    if (l_trace) l_trace[nchunks] = l;
  }
  for (long i = 0; i < n; ++i) p[i] = (l > 0.0) ? exp(x[i] - m) / l : 0.0;
  return nchunks;
}

/*
 * Standard three-step attention for one block of query rows of one head
 * [P3 §"Le problème": S = Q K^T, P = softmax(S), O = P V;  P1 §"Het fysieke
 * knelpunt": the same three steps;  P4 "Apa itu FlashAttention?":
 * softmax(Q K^T / sqrt(d)) V].
 *
 *   q [nq, d], k [nk, d], v [nk, d]  ->  o [nq, d], lse [nq], rows r0..r1-1
 *   qpos[r] (may be NULL: r) is the sequence position of query row r, used
 *   only by the causal mask.
 *
 * Step 1 forms all scores of the block, step 2 turns each score row into
 * probabilities (and its lse), step 3 multiplies by V.  s and p are scratch
 * of (r1 - r0) * nk doubles each.
 */
static void oracle_fwd_rows(const double* q, const long* qpos, long r0, long r1,
                            const double* k, const double* v, long nk, long d,
                            double scale, int causal, long window, double* o, double* lse,
                            double* s, double* p) {
  /* step 1: S = scale * Q K^T, masked entries = -inf */
  for (long r = r0; r < r1; ++r) {
    long i = qpos ? qpos[r] : r;
    double* srow = s + (r - r0) * nk;
    for (long j = 0; j < nk; ++j) {
      if (!oracle_visible(i, j, causal, window)) { srow[j] = -INFINITY; continue; }
      double acc = 0.0;
      for (long c = 0; c < d; ++c) acc += q[r * d + c] * k[j * d + c];
      srow[j] = scale * acc;
    }
  }
  /* step 2: P = softmax(S) row by row; lse = m + ln(sum_j e^{s_j - m}) */
  for (long r = r0; r < r1; ++r) {
    const double* srow = s + (r - r0) * nk;
    oracle_softmax(srow, nk, p + (r - r0) * nk);
    double m = -INFINITY;
    for (long j = 0; j < nk; ++j) if (srow[j] > m) m = srow[j];
    if (m == -INFINITY) { lse[r] = -INFINITY; continue; }
    double sum = 0.0;
    for (long j = 0; j < nk; ++j) sum += exp(srow[j] - m);
    lse[r] = m + log(sum);
  }
  /* step 3: O = P V */
  for (long r = r0; r < r1; ++r) {
    const double* prow = p + (r - r0) * nk;
    double* orow = o + r * d;
    for (long c = 0; c < d; ++c) orow[c] = 0.0;
    for (long j = 0; j < nk; ++j) {
      double pj = prow[j];
      if (pj == 0.0) continue;
      for (long c = 0; c < d; ++c) orow[c] += pj * v[j * d + c];
    }
  }
}

/*
 * Forward over B x H query heads.  q [B, H, nq, d]; k, v [B, Hkv, nk, d];
 * o [B, H, nq, d]; lse [B, H, nq].  Query head h of batch b reads key/value
 * head b * Hkv + h / (H / Hkv) (Hkv = H is plain multi-head attention).
 * qpos (may be NULL) applies to every head.  Independent (head, row block)
 * tasks run in parallel.
 */
int oracle_attn_fwd_w(const double* q, const double* k, const double* v,
                      double* o, double* lse, long B, long H, long Hkv, long nq, long nk,
                      long d, double scale, int causal, long window, const long* qpos,
                      int nthreads) {
  if (!q || !k || !v || !o || !lse || B < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || nq < 0 ||
      nk < 0 || d <= 0)
    return 1;
  oracle_set_threads(nthreads);
  long nblk = (nq + ORACLE_ROWS_PER_TASK - 1) / ORACLE_ROWS_PER_TASK;
  long ntask = B * H * nblk;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * ORACLE_ROWS_PER_TASK * (size_t)nk + 8);
    double* p = (double*)malloc(sizeof(double) * ORACLE_ROWS_PER_TASK * (size_t)nk + 8);
    if (!s || !p) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic)
    for (long t = 0; t < ntask; ++t) {
      if (!s || !p) continue;
      long qh = t / nblk, r0 = (t % nblk) * ORACLE_ROWS_PER_TASK;
      long b = qh / H, h = qh % H;
      long kvh = b * Hkv + h / (H / Hkv);
      long r1 = r0 + ORACLE_ROWS_PER_TASK < nq ? r0 + ORACLE_ROWS_PER_TASK : nq;
      oracle_fwd_rows(q + qh * nq * d, qpos, r0, r1, k + kvh * nk * d, v + kvh * nk * d, nk, d,
                      scale, causal, window, o + qh * nq * d, lse + qh * nq, s, p);
    }
    free(s);
    free(p);
  }
  return failed ? 2 : 0;
}

/* Forward over BH independent heads (multi-head, no window). */
int oracle_attn_fwd(const double* q, const double* k, const double* v,
                    double* o, double* lse, long BH, long nq, long nk, long d,
                    double scale, int causal, const long* qpos, int nthreads) {
  if (BH == 0) return (!q || !k || !v || !o || !lse || nq < 0 || nk < 0 || d <= 0) ? 1 : 0;
  return oracle_attn_fwd_w(q, k, v, o, lse, 1, BH, BH, nq, nk, d, scale, causal, 0, qpos,
                           nthreads);
}

/*
 * Decode: one query token per head against the whole key/value history, no
 * mask [P1 §"Interactie met de KV-cache tijdens inferentie": N_q = 1 while K
 * and V span the history].  The oracle does not split the history: splitting
 * is the GPU method's business.  q [BH, d]; k, v [BH, nkv, d]; o [BH, d];
 * lse [BH].
 */
int oracle_attn_decode(const double* q, const double* k, const double* v,
                       double* o, double* lse, long BH, long nkv, long d,
                       double scale, int nthreads) {
  return oracle_attn_fwd(q, k, v, o, lse, BH, 1, nkv, d, scale, 0, NULL, nthreads);
}

/* Decode with grouped key/value heads: q [B, H, d]; k, v [B, Hkv, nkv, d]. */
int oracle_attn_decode_w(const double* q, const double* k, const double* v,
                         double* o, double* lse, long B, long H, long Hkv, long nkv, long d,
                         double scale, int nthreads) {
  return oracle_attn_fwd_w(q, k, v, o, lse, B, H, Hkv, 1, nkv, d, scale, 0, 0, NULL, nthreads);
}

/*
 * Tiled forward with online softmax, one head, in the order the pages give
 * [P1 §"Algoritmische kern in pseudocode"; P3 §"Mécanisme"]: Q is cut into
 * blocks of br rows, K and V into blocks of bc rows; for each Q block, O,
 * the running sum l and running max m start at 0, 0, -inf; for every K/V
 * block the scores S = scale * Q_i K_j^T are formed, m_new = max(m, rowmax S),
 * P = e^{S - m_new}, l = e^{m - m_new} l + rowsum P and
 * O = diag(e^{m - m_new}) O + P V_j; after the last block O = diag(1/l) O.
 * Used only to check that tiling changes nothing but rounding [P4 Step 6].
 */
int oracle_attn_fwd_tiled(const double* q, const double* k, const double* v,
                          double* o, double* lse, long nq, long nk, long d,
                          double scale, int causal, long br, long bc) {
  if (!q || !k || !v || !o || !lse || br <= 0 || bc <= 0) return 1;
  double* s = (double*)malloc(sizeof(double) * br * bc);
  double* m = (double*)malloc(sizeof(double) * br);
  double* l = (double*)malloc(sizeof(double) * br);
  for (long i0 = 0; i0 < nq; i0 += br) {
    long i1 = i0 + br < nq ? i0 + br : nq;
    for (long r = i0; r < i1; ++r) {
      m[r - i0] = -INFINITY;
      l[r - i0] = 0.0;
      for (long c = 0; c < d; ++c) o[r * d + c] = 0.0;
    }
    for (long j0 = 0; j0 < nk; j0 += bc) {
      long j1 = j0 + bc < nk ? j0 + bc : nk;
      for (long r = i0; r < i1; ++r) {
        double* srow = s + (r - i0) * bc;
        double rowmax = -INFINITY;
        for (long j = j0; j < j1; ++j) {
          double acc = -INFINITY;
          if (oracle_visible(r, j, causal, 0)) {
            acc = 0.0;
            for (long c = 0; c < d; ++c) acc += q[r * d + c] * k[j * d + c];
            acc *= scale;
          }
          srow[j - j0] = acc;
          if (acc > rowmax) rowmax = acc;
        }
        double m_old = m[r - i0];
        double m_new = m_old > rowmax ? m_old : rowmax;
        if (m_new == -INFINITY) continue; /* nothing visible yet */
        double alpha = (m_old == -INFINITY) ? 0.0 : exp(m_old - m_new);
        double rowsum = 0.0;
        for (long c = 0; c < d; ++c) o[r * d + c] *= alpha;
        for (long j = j0; j < j1; ++j) {
          double pj = exp(srow[j - j0] - m_new);
          rowsum += pj;
          if (pj == 0.0) continue;
          for (long c = 0; c < d; ++c) o[r * d + c] += pj * v[j * d + c];
        }
        l[r - i0] = alpha * l[r - i0] + rowsum;
        m[r - i0] = m_new;
      }
    }
    for (long r = i0; r < i1; ++r) {
      double lr = l[r - i0];
      if (lr > 0.0) {
        for (long c = 0; c < d; ++c) o[r * d + c] /= lr;
        lse[r] = m[r - i0] + log(lr);
      } else {
        for (long c = 0; c < d; ++c) o[r * d + c] = 0.0;
        lse[r] = -INFINITY;
      }
    }
  }
  free(s);
  free(m);
  free(l);
  return 0;
}

/*
 * Merge of per-chunk summaries of one row: chunk c carries its normalised
 * output o_c (d values) and its log-sum-exp lse_c.  This is the online
 * softmax update [P4 Step 4] applied to whole chunks: with M = max_c lse_c
 * and w_c = e^{lse_c - M}, the row's output is sum_c w_c o_c / sum_c w_c and
 * its lse is M + ln(sum_c w_c).  A chunk with lse_c = -inf has weight 0.
 * Used only to check the split-history decode's semantics.
 */
int oracle_lse_merge(const double* o_parts, const double* lse_parts, long nparts,
                     long d, double* o, double* lse) {
  if (!o_parts || !lse_parts || !o || !lse || nparts <= 0) return 1;
  double big = -INFINITY;
  for (long c = 0; c < nparts; ++c) if (lse_parts[c] > big) big = lse_parts[c];
  for (long x = 0; x < d; ++x) o[x] = 0.0;
  if (big == -INFINITY) { *lse = -INFINITY; return 0; }
  double wsum = 0.0;
  for (long c = 0; c < nparts; ++c) {
    double w = exp(lse_parts[c] - big);
    wsum += w;
    if (w == 0.0) continue;
    for (long x = 0; x < d; ++x) o[x] += w * o_parts[c * d + x];
  }
  for (long x = 0; x < d; ++x) o[x] /= wsum;
  *lse = big + log(wsum);
  return 0;
}

/*
 * Backward pass of the three-step definition, one head.  The pages fix only
 * that P is rebuilt from the inputs and the saved statistics rather than
 * stored [P1 §"Geheugencomplexiteit: van O(N²) naar O(N)"; P3 §"Backward
 * pass"]; the gradients themselves are the plain calculus of
 * O = softmax(scale * Q K^T) V for an upstream gradient dO:
 *   dV = P^T dO
 *   dP = dO V^T
 *   D_i = sum_j P_ij dP_ij                (row dot product, by definition)
 *   dS = P o (dP - D 1^T)                 (softmax Jacobian, o = elementwise)
 *   dQ = scale * dS K
 *   dK = scale * dS^T Q
 * Masked entries have P = 0 and so contribute nothing.  P is rebuilt here
 * from the definition in float64 (it does not use any saved statistic).
 * Scratch: two n x n double matrices per head.  Returns 0, or 2 if a
 * thread's row buffer could not be allocated (outputs then undefined).
 */
static int oracle_bwd_head(const double* q, const double* k, const double* v,
                            const double* dout, double* dq, double* dk, double* dv,
                            double* drow, long n, long d, double scale, int causal, long window,
                            double* P, double* dS) {
  int failed = 0;
  /* rebuild P row by row from its definition */
#pragma omp parallel
  {
    double* srow = (double*)malloc(sizeof(double) * (size_t)n + 8);
    if (!srow) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (long i = 0; i < n; ++i) {
      if (!srow) continue;
      for (long j = 0; j < n; ++j) {
        if (!oracle_visible(i, j, causal, window)) { srow[j] = -INFINITY; continue; }
        double acc = 0.0;
        for (long c = 0; c < d; ++c) acc += q[i * d + c] * k[j * d + c];
        srow[j] = scale * acc;
      }
      oracle_softmax(srow, n, P + i * n);
    }
    free(srow);
  }
  if (failed) return 2;
  /* dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P o (dP - D) */
#pragma omp parallel for schedule(dynamic, 16)
  for (long i = 0; i < n; ++i) {
    double* dsrow = dS + i * n;
    for (long j = 0; j < n; ++j) {
      double acc = 0.0;
      if (oracle_visible(i, j, causal, window))
        for (long c = 0; c < d; ++c) acc += dout[i * d + c] * v[j * d + c];
      dsrow[j] = acc; /* dP for now */
    }
    double di = 0.0;
    for (long j = 0; j < n; ++j) di += P[i * n + j] * dsrow[j];
    if (drow) drow[i] = di;
    for (long j = 0; j < n; ++j) dsrow[j] = P[i * n + j] * (dsrow[j] - di);
  }
  /* dQ = scale * dS K */
#pragma omp parallel for schedule(dynamic, 16)
  for (long i = 0; i < n; ++i) {
    for (long c = 0; c < d; ++c) dq[i * d + c] = 0.0;
    for (long j = 0; j < n; ++j) {
      double w = dS[i * n + j];
      if (w == 0.0) continue;
      for (long c = 0; c < d; ++c) dq[i * d + c] += w * k[j * d + c];
    }
    for (long c = 0; c < d; ++c) dq[i * d + c] *= scale;
  }
  /* dK = scale * dS^T Q and dV = P^T dO, one key row j at a time */
#pragma omp parallel for schedule(dynamic, 16)
  for (long j = 0; j < n; ++j) {
    for (long c = 0; c < d; ++c) { dk[j * d + c] = 0.0; dv[j * d + c] = 0.0; }
    for (long i = 0; i < n; ++i) {
      double ws = dS[i * n + j], wp = P[i * n + j];
      if (ws != 0.0)
        for (long c = 0; c < d; ++c) dk[j * d + c] += ws * q[i * d + c];
      if (wp != 0.0)
        for (long c = 0; c < d; ++c) dv[j * d + c] += wp * dout[i * d + c];
    }
    for (long c = 0; c < d; ++c) dk[j * d + c] *= scale;
  }
  return 0;
}

/*
 * Backward over B x H query heads with grouped key/value heads.
 * q, dout, dq: [B, H, n, d]; k, v, dk, dv: [B, Hkv, n, d]; drow (may be
 * NULL): [B, H, n].  A key/value head is an input of each query head of its
 * group, so its gradient is the sum of the group's per-head gradients
 * (chain rule), added here in head order.
 * Returns 0 on success, 1 on bad arguments, 2 if scratch allocation failed.
 */
int oracle_attn_bwd_w(const double* q, const double* k, const double* v,
                      const double* dout, double* dq, double* dk, double* dv,
                      double* drow, long B, long H, long Hkv, long n, long d, double scale,
                      int causal, long window, int nthreads) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 0 || H < 1 || Hkv < 1 ||
      H % Hkv != 0 || n < 0 || d <= 0)
    return 1;
  oracle_set_threads(nthreads);
  double* P = (double*)malloc(sizeof(double) * (size_t)n * (size_t)n + 8);
  double* dS = (double*)malloc(sizeof(double) * (size_t)n * (size_t)n + 8);
  double* gk = (double*)malloc(sizeof(double) * (size_t)n * (size_t)d + 8);
  double* gv = (double*)malloc(sizeof(double) * (size_t)n * (size_t)d + 8);
  if (!P || !dS || !gk || !gv) { free(P); free(dS); free(gk); free(gv); return 2; }
  memset(dk, 0, sizeof(double) * (size_t)(B * Hkv) * n * d);
  memset(dv, 0, sizeof(double) * (size_t)(B * Hkv) * n * d);
  for (long b = 0; b < B; ++b)
    for (long h = 0; h < H; ++h) {
      size_t qoff = (size_t)(b * H + h) * n * d;
      size_t kvoff = (size_t)(b * Hkv + h / (H / Hkv)) * n * d;
      if (oracle_bwd_head(q + qoff, k + kvoff, v + kvoff, dout + qoff, dq + qoff, gk, gv,
                          drow ? drow + (b * H + h) * n : NULL, n, d, scale, causal, window, P,
                          dS) != 0) {
        free(P); free(dS); free(gk); free(gv);
        return 2;
      }
      for (long e = 0; e < n * d; ++e) {
        dk[kvoff + e] += gk[e];
        dv[kvoff + e] += gv[e];
      }
    }
  free(P);
  free(dS);
  free(gk);
  free(gv);
  return 0;
}

/* Backward over BH independent heads (multi-head, no window). */
int oracle_attn_bwd(const double* q, const double* k, const double* v,
                    const double* dout, double* dq, double* dk, double* dv,
                    double* drow, long BH, long n, long d, double scale, int causal,
                    int nthreads) {
  if (BH == 0) return (!q || !k || !v || !dout || !dq || !dk || !dv || n < 0 || d <= 0) ? 1 : 0;
  return oracle_attn_bwd_w(q, k, v, dout, dq, dk, dv, drow, 1, BH, BH, n, d, scale, causal, 0,
                           nthreads);
}
