/* A driver for the float64 oracle (oracle/oracle.c), built by the CPU test suite together
 * with oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * It calls every exported oracle function on small inputs -- including the edge cases the
 * oracle defines: empty query or key sets, rows with no visible key, a sliding window, grouped
 * key/value heads, one-key histories -- so that any out-of-bounds access, use of freed memory
 * or undefined arithmetic in the oracle stops the run.  Each call is also checked against an
 * identity the mathematics fixes (rows of P sum to 1, chunked online softmax equals the plain
 * softmax, the tiled forward equals the three-step forward, a merge of chunk summaries equals
 * the whole row, the backward's column sums), so the run is not only memory-clean but right.
 * Prints one line per check; exits non-zero on any failure.  Needs no GPU. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's exported functions (oracle.c has no header; these are its definitions). */
int oracle_max_threads(void);
void oracle_softmax(const double* x, long n, double* p);
long oracle_softmax_online(const double* x, long n, long chunk, double* p, double* m_trace,
                           double* l_trace);
int oracle_attn_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                    long BH, long nq, long nk, long d, double scale, int causal, const long* qpos,
                    int nthreads);
int oracle_attn_fwd_w(const double* q, const double* k, const double* v, double* o, double* lse,
                      long B, long H, long Hkv, long nq, long nk, long d, double scale, int causal,
                      long window, const long* qpos, int nthreads);
int oracle_attn_decode(const double* q, const double* k, const double* v, double* o, double* lse,
                       long BH, long nkv, long d, double scale, int nthreads);
int oracle_attn_decode_w(const double* q, const double* k, const double* v, double* o,
                         double* lse, long B, long H, long Hkv, long nkv, long d, double scale,
                         int nthreads);
int oracle_attn_fwd_tiled(const double* q, const double* k, const double* v, double* o,
                          double* lse, long nq, long nk, long d, double scale, int causal, long br,
                          long bc);
int oracle_lse_merge(const double* o_parts, const double* lse_parts, long nparts, long d,
                     double* o, double* lse);
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv, double* drow, long BH, long n, long d,
                    double scale, int causal, int nthreads);
int oracle_attn_bwd_w(const double* q, const double* k, const double* v, const double* dout,
                      double* dq, double* dk, double* dv, double* drow, long B, long H, long Hkv,
                      long n, long d, double scale, int causal, long window, int nthreads);

static int failures = 0;

static void check(const char* what, int ok) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

static unsigned long long rng_state = 88172645463325252ULL;
static double uniform(void) { /* xorshift64, mapped to [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double* filled(long n) {
  double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (long i = 0; i < n; ++i) a[i] = uniform() * 2.0;
  return a;
}
static double max_abs_diff(const double* a, const double* b, long n) {
  double m = 0.0;
  for (long i = 0; i < n; ++i) {
    double d = fabs(a[i] - b[i]);
    if (d > m || d != d) m = d;
  }
  return m;
}

int main(void) {
  printf("oracle threads %d\n", oracle_max_threads());

  /* softmax and chunked online softmax on the eight-score example */
  const double x8[8] = {1.2, 3.0, 0.4, 2.1, 4.5, 1.8, 3.6, 0.9};
  double p[8], po[8], mt[8], lt[8];
  oracle_softmax(x8, 8, p);
  double s = 0.0;
  for (int i = 0; i < 8; ++i) s += p[i];
  check("softmax row sums to 1", fabs(s - 1.0) < 1e-15);
  int online_ok = 1;
  for (long c = 1; c <= 8; ++c) {
    long nch = oracle_softmax_online(x8, 8, c, po, mt, lt);
    online_ok &= nch == (8 + c - 1) / c && max_abs_diff(p, po, 8) < 1e-15;
  }
  check("online softmax equals softmax for chunks 1..8", online_ok);
  check("online softmax of an empty row", oracle_softmax_online(x8, 0, 3, po, mt, lt) == 0);
  const double masked[3] = {-INFINITY, -INFINITY, -INFINITY};
  oracle_softmax(masked, 3, p);
  check("fully masked row gives zeros", p[0] == 0.0 && p[1] == 0.0 && p[2] == 0.0);

  /* forward with grouped heads and a window; tiled forward; decode; merge */
  const long B = 2, H = 4, Hkv = 2, n = 37, d = 8;
  const double scale = 1.0 / sqrt((double)d);
  double* q = filled(B * H * n * d);
  double* k = filled(B * Hkv * n * d);
  double* v = filled(B * Hkv * n * d);
  double* o = filled(B * H * n * d);
  double* lse = filled(B * H * n);
  check("fwd_w grouped causal window 5",
        oracle_attn_fwd_w(q, k, v, o, lse, B, H, Hkv, n, n, d, scale, 1, 5, NULL, 0) == 0);
  double* o2 = filled(n * d);
  double* l2 = filled(n);
  check("tiled fwd 5 x 7 tiles", oracle_attn_fwd_tiled(q, k, v, o2, l2, n, n, d, scale, 1, 5, 7) == 0);
  double* o3 = filled(n * d);
  double* l3 = filled(n);
  check("fwd one head causal", oracle_attn_fwd(q, k, v, o3, l3, 1, n, n, d, scale, 1, NULL, 1) == 0);
  check("tiled fwd equals three-step fwd",
        max_abs_diff(o2, o3, n * d) < 1e-13 && max_abs_diff(l2, l3, n) < 1e-13);
  long qpos[3] = {0, 17, 36};
  double qsel[3 * 8];
  for (int r = 0; r < 3; ++r) memcpy(qsel + r * d, q + qpos[r] * d, sizeof(double) * d);
  double* oq = filled(3 * d);
  double* lq = filled(3);
  check("fwd at chosen query positions",
        oracle_attn_fwd(qsel, k, v, oq, lq, 1, 3, n, d, scale, 1, qpos, 0) == 0 &&
            max_abs_diff(oq + d, o3 + 17 * d, d) < 1e-14 && max_abs_diff(lq + 2, l3 + 36, 1) < 1e-14);
  double* od = filled(B * H * d);
  double* ld = filled(B * H);
  check("decode_w grouped", oracle_attn_decode_w(q, k, v, od, ld, B, H, Hkv, n, d, scale, 0) == 0);
  double* of = filled(B * H * d);
  double* lf = filled(B * H);
  /* the decode query of (b, h) is row 0 of q's head (b, h) when nq = 1 */
  double* q1 = filled(B * H * d);
  for (long bh = 0; bh < B * H; ++bh) memcpy(q1 + bh * d, q + bh * n * d, sizeof(double) * d);
  check("decode_w on single rows",
        oracle_attn_decode_w(q1, k, v, od, ld, B, H, Hkv, n, d, scale, 0) == 0 &&
            oracle_attn_fwd_w(q1, k, v, of, lf, B, H, Hkv, 1, n, d, scale, 0, 0, NULL, 0) == 0 &&
            max_abs_diff(od, of, B * H * d) == 0.0 && max_abs_diff(ld, lf, B * H) == 0.0);
  double* od1 = filled(d);
  double* ld1 = filled(1);
  check("decode one head", oracle_attn_decode(q1, k, v, od1, ld1, 1, n, d, scale, 1) == 0);
  /* three chunk summaries of head 0's history merge to the whole row */
  double parts_o[3 * 8], parts_l[3], mo[8], ml;
  const long cuts[4] = {0, 10, 11, 37};
  int merge_calls_ok = 1;
  for (int c = 0; c < 3; ++c)
    merge_calls_ok &= oracle_attn_decode(q1, k + cuts[c] * d, v + cuts[c] * d, parts_o + c * d,
                                         parts_l + c, 1, cuts[c + 1] - cuts[c], d, scale, 1) == 0;
  merge_calls_ok &= oracle_lse_merge(parts_o, parts_l, 3, d, mo, &ml) == 0;
  check("merge of chunk summaries equals the whole row",
        merge_calls_ok && max_abs_diff(mo, od1, d) < 1e-14 && fabs(ml - ld1[0]) < 1e-14);
  parts_l[1] = -INFINITY; /* an empty chunk has weight zero */
  check("merge with an empty chunk", oracle_lse_merge(parts_o, parts_l, 3, d, mo, &ml) == 0);

  /* edge cases the oracle defines */
  check("fwd with no query rows", oracle_attn_fwd(q, k, v, o, lse, 1, 0, n, d, scale, 1, NULL, 0) == 0);
  double* oe = filled(4 * d);
  double* le = filled(4);
  check("fwd with no keys: o = 0, lse = -inf",
        oracle_attn_fwd(q, k, v, oe, le, 1, 4, 0, d, scale, 0, NULL, 0) == 0 && oe[0] == 0.0 &&
            le[3] == -INFINITY);
  check("decode of a one-key history: o = v",
        oracle_attn_decode(q1, k, v, od1, ld1, 1, 1, d, scale, 1) == 0 && max_abs_diff(od1, v, d) == 0.0);
  check("bad arguments are refused",
        oracle_attn_fwd_w(q, k, v, o, lse, B, 3, 2, n, n, d, scale, 0, 0, NULL, 0) == 1 &&
            oracle_attn_fwd_tiled(q, k, v, o2, l2, n, n, d, scale, 1, 0, 7) == 1 &&
            oracle_lse_merge(parts_o, parts_l, 0, d, mo, &ml) == 1 &&
            oracle_attn_bwd_w(NULL, k, v, q, o, o, o, NULL, 1, 1, 1, n, d, scale, 0, 0, 0) == 1);

  /* backward: grouped heads with a window, then plain heads */
  const long nb = 11, db = 4;
  double* bq = filled(B * H * nb * db);
  double* bk = filled(B * Hkv * nb * db);
  double* bv = filled(B * Hkv * nb * db);
  double* bdo = filled(B * H * nb * db);
  double* bdq = filled(B * H * nb * db);
  double* bdk = filled(B * Hkv * nb * db);
  double* bdv = filled(B * Hkv * nb * db);
  double* bdr = filled(B * H * nb);
  check("bwd_w grouped causal window 3",
        oracle_attn_bwd_w(bq, bk, bv, bdo, bdq, bdk, bdv, bdr, B, H, Hkv, nb, db, 0.5, 1, 3, 0) == 0);
  /* column sums: sum_j dK_j = 0 (rows of dS sum to 0); sum_j dV_j = sum over the group's
   * query heads of sum_i dO_i (rows of P sum to 1) */
  int sums_ok = 1;
  for (long g = 0; g < B * Hkv; ++g)
    for (long c = 0; c < db; ++c) {
      double sk = 0.0, sv = 0.0, sdo = 0.0;
      for (long j = 0; j < nb; ++j) {
        sk += bdk[(g * nb + j) * db + c];
        sv += bdv[(g * nb + j) * db + c];
      }
      const long b = g / Hkv, hk = g % Hkv, grp = H / Hkv;
      for (long h = hk * grp; h < (hk + 1) * grp; ++h)
        for (long i = 0; i < nb; ++i) sdo += bdo[((b * H + h) * nb + i) * db + c];
      sums_ok &= fabs(sk) < 1e-12 && fabs(sv - sdo) < 1e-12;
    }
  check("bwd column sums (dK to 0, dV to the group's dO)", sums_ok);
  check("bwd plain heads, no row terms",
        oracle_attn_bwd(bq, bk, bv, bdo, bdq, bdk, bdv, NULL, 2, nb, db, 0.5, 0, 1) == 0);
  check("bwd with no rows", oracle_attn_bwd(bq, bk, bv, bdo, bdq, bdk, bdv, bdr, 1, 0, db, 0.5, 1, 0) == 0);
  check("bwd with no heads", oracle_attn_bwd(bq, bk, bv, bdo, bdq, bdk, bdv, bdr, 0, nb, db, 0.5, 1, 0) == 0);

  free(q); free(k); free(v); free(o); free(lse); free(o2); free(l2); free(o3); free(l3);
  free(oq); free(lq); free(od); free(ld); free(of); free(lf); free(q1); free(od1); free(ld1);
  free(oe); free(le); free(bq); free(bk); free(bv); free(bdo); free(bdq); free(bdk); free(bdv);
  free(bdr);
  printf("%d failure(s)\n", failures);
  return failures != 0;
}
