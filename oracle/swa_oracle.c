/*
 * swa_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A plain, slow, fp64 CPU implementation of exact causal sliding-window
 * attention with attention sinks.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the HIP library; it is written directly from the
 * definitions on the source pages:
 *
 *  [P3] "Sliding Window and Sparse Attention, from Longformer to CSA2"
 *       section 1 (attention = softmax(Q K^T / sqrt(d)) V, causal j <= i),
 *       section 2 (the window: key positions i-w+1 .. i, w of them counting
 *       i itself; sinks: positions 0 .. g-1 are kept readable for good),
 *       section 10 glossary "LSE" (the softmax normaliser).
 *  [P4] "Local and Sparse Attention: Reading Fewer Token Positions"
 *       Figure 1 (window of 3 = current position plus the two before it),
 *       the paragraph after Figure 1 (excluded positions get -inf before the
 *       softmax; a zero score is a different computation),
 *       Figure 2 (window united with a fixed anchor position; a position in
 *       both sets is read once; no future position is read).
 *
 * Every function here evaluates the definition directly: the attended set
 * A_i is decided by a per-pair predicate, every score of a row is formed,
 * excluded scores are -inf, then a two-pass max / exp-sum / weighted sum.
 * There is no tiling, no online recurrence and no reordering.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: -inf and exp(-inf)=0
 * semantics are relied on).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Attended-set predicate.  Query position i reads key position j iff
 *   j <= i                         (causal, [P3] s1; [P4] Fig. 2: no future)
 *   and ( i-w+1 <= j               (window of w keys incl. i, [P3] s2, [P4] Fig. 1)
 *         or j < g )               (sink / anchor positions, [P3] s2, [P4] Fig. 2)
 * The union is a set, so a key in both parts is counted once ([P4] Fig. 2). */
int swa_oracle_attended(long i, long j, long w, long g)
{
    if (j < 0 || j > i) return 0;
    if (j >= i - w + 1) return 1;
    if (j < g) return 1;
    return 0;
}

/* |A_i| by scanning every candidate key position 0..i. */
long swa_oracle_row_count(long i, long w, long g)
{
    long c = 0;
    for (long j = 0; j <= i; ++j) c += swa_oracle_attended(i, j, w, g);
    return c;
}

/* Total attended (query, key) pairs of an n-token sequence: sum of |A_i|.
 * [P4] Figure 1 prints 36 for full causal and 21 for w=3 at n=8. */
long swa_oracle_pair_count(long n, long w, long g)
{
    long c = 0;
    for (long i = 0; i < n; ++i) c += swa_oracle_row_count(i, w, g);
    return c;
}

/* Dense n x n connectivity grid, row = query, column = key, 1 = attended. */
int swa_oracle_mask(long n, long w, long g, unsigned char *out)
{
    if (n < 0 || !out) return -1;
    for (long i = 0; i < n; ++i)
        for (long j = 0; j < n; ++j)
            out[i * n + j] = (unsigned char)swa_oracle_attended(i, j, w, g);
    return 0;
}

static double dot(const double *a, const double *b, long d)
{
    double s = 0.0;
    for (long c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

/* One query row over an explicit list of candidate keys.
 *   qi         : the query vector [d]
 *   kp[t]      : key position of candidate t (skipped if < 0)
 *   krow/vrow  : key / value vectors of candidate t, [nk][d]
 * Scores:  s_t = scale * q.k_t + beta * [kp_t < g]  if kp_t in A_i, else -inf
 * ([P3] s1 for scale = 1/sqrt(d) and the softmax; [P4] after Fig. 1 for the
 * -inf).  The sink offset beta is an additive bias on the scaled score of
 * every attended key at a position below g.
 * Then m = max s, l = sum exp(s - m), o = sum exp(s - m) v / l, lse = m + ln l.
 * s is caller-provided scratch of nk doubles. */
static void attend_row(const double *qi, long i, const long *kp, const double *krow,
                       const double *vrow, long nk, long d, long w, long g,
                       double scale, double beta, double *s, double *o, double *lse)
{
    double m = -INFINITY;
    for (long t = 0; t < nk; ++t) {
        long j = kp[t];
        if (j >= 0 && swa_oracle_attended(i, j, w, g)) {
            s[t] = scale * dot(qi, krow + t * d, d) + (j < g ? beta : 0.0);
        } else {
            s[t] = -INFINITY;
        }
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (long t = 0; t < nk; ++t) l += exp(s[t] - m);
    for (long c = 0; c < d; ++c) o[c] = 0.0;
    for (long t = 0; t < nk; ++t) {
        double p = exp(s[t] - m);
        if (p == 0.0) continue;
        const double *vt = vrow + t * d;
        for (long c = 0; c < d; ++c) o[c] += p * vt[c];
    }
    for (long c = 0; c < d; ++c) o[c] /= l;
    *lse = m + log(l);
}

/* Prefill over a whole sequence.
 *   q, k, v : [bh][n][d] fp64 (bh = batch*heads independent slices)
 *   rows    : query rows to evaluate (every slice), or NULL for all n rows
 *   o       : [bh][nrows][d],  lse : [bh][nrows] (may be NULL)
 * Row i forms a score for every key position 0..i (a dense causal row); the
 * predicate turns the excluded ones into -inf.
 * Returns 0, or -1 on bad arguments / allocation failure. */
int swa_oracle_prefill(const double *q, const double *k, const double *v,
                       long bh, long n, long d, long w, long g,
                       double scale, double beta, const long *rows, long nrows,
                       double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !o || bh < 0 || n < 0 || d < 1 || w < 1 || g < 0) return -1;
    if (!rows) nrows = n;
    for (long r = 0; r < nrows; ++r) {
        long i = rows ? rows[r] : r;
        if (i < 0 || i >= n) return -1;
    }
    long *pos = (long *)malloc(sizeof(long) * (size_t)(n > 0 ? n : 1));
    if (!pos) return -1;
    for (long j = 0; j < n; ++j) pos[j] = j;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double *orow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !orow) {
#pragma omp atomic write
            bad = 1;
        }
        /* every thread reaches the work-sharing loop; one without scratch skips */
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (long b = 0; b < bh; ++b) {
            for (long r = 0; r < nrows; ++r) {
                if (!s || !orow) continue;
                long i = rows ? rows[r] : r;
                const double *base_k = k + (size_t)b * n * d;
                const double *base_v = v + (size_t)b * n * d;
                double l_out;
                /* candidates: key positions 0..i, i.e. the causal row */
                attend_row(q + ((size_t)b * n + i) * d, i, pos, base_k, base_v,
                           i + 1, d, w, g, scale, beta, s, orow, &l_out);
                memcpy(o + ((size_t)b * nrows + r) * d, orow, sizeof(double) * (size_t)d);
                if (lse) lse[(size_t)b * nrows + r] = l_out;
            }
        }
        free(s);
        free(orow);
    }
    free(pos);
    return bad ? -1 : 0;
}

static int cmp_long(const void *a, const void *b)
{
    long x = *(const long *)a, y = *(const long *)b;
    return (x > y) - (x < y);
}

/* Decode: one query at position p per unit, over the logical sequence.
 *   q    : [units][d]
 *   p    : [units] query positions
 *   kpos : [units][nk] logical positions of the supplied key/value rows
 *          (entries < 0 are padding and ignored)
 *   k, v : [units][nk][d]
 * The caller supplies key/value rows by logical position; the oracle applies
 * the attended-set predicate itself and refuses (returns -2) a unit whose
 * supplied rows do not cover A_p exactly once, or that supplies a position
 * twice.  It never looks at a cache layout.
 * Returns 0, -1 on bad arguments, -2 on an incomplete / duplicated key set. */
int swa_oracle_decode(const double *q, const long *p, const long *kpos,
                      const double *k, const double *v, long units, long nk, long d,
                      long w, long g, double scale, double beta,
                      double *o, double *lse, int nthreads)
{
    if (!q || !p || !kpos || !k || !v || !o || units < 0 || nk < 1 || d < 1 || w < 1 || g < 0)
        return -1;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)nk);
        long *sorted = (long *)malloc(sizeof(long) * (size_t)nk);
        if (!s || !sorted) {
#pragma omp atomic write
            bad = -1;
        }
        /* every thread reaches the work-sharing loop; one without scratch skips */
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!s || !sorted) continue;
            const long *kp = kpos + (size_t)u * nk;
            long pu = p[u];
            /* completeness: every attended position present exactly once */
            long supplied = 0, dup = 0;
            memcpy(sorted, kp, sizeof(long) * (size_t)nk);
            qsort(sorted, (size_t)nk, sizeof(long), cmp_long);
            for (long t = 0; t < nk; ++t) {
                if (sorted[t] < 0) continue;
                if (t > 0 && sorted[t - 1] == sorted[t]) dup = 1;
                supplied += swa_oracle_attended(pu, sorted[t], w, g);
            }
            if (dup || pu < 0 || supplied != swa_oracle_row_count(pu, w, g)) {
#pragma omp atomic write
                bad = -2;
                continue;
            }
            double l_out;
            attend_row(q + (size_t)u * d, pu, kp, k + (size_t)u * nk * d,
                       v + (size_t)u * nk * d, nk, d, w, g, scale, beta, s,
                       o + (size_t)u * d, &l_out);
            if (lse) lse[u] = l_out;
        }
        free(s);
        free(sorted);
    }
    return bad;
}

int swa_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
