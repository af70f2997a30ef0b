// Host-only checks of the fp64 oracle (oracle/swa_oracle.c) and of the prefill
// tile scheduler (block_sparse_causal_band_amd/csrc/schedule.h), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py
// and run as an executable of its own.  Test infrastructure only.
//
// The checks are the ones the Python suite runs through ctypes, restated here
// so that every memory access and every integer operation of both host codes
// runs under the sanitizers:
//  * oracle: the counts printed with Figure 1 of "Local and Sparse Attention:
//    Reading Fewer Token Positions" (36 causal, 21 with a window of 3 at 8
//    tokens) and the closed form n w - w(w-1)/2; the read sets of Figures 1
//    and 2 of that page; a window at least n long equal to plain causal
//    attention (written out below); a window of 1 returning V; a zero query
//    giving the bias-weighted mean of the attended values; decode over the
//    logical sequence equal to the prefill row; incomplete key sets refused;
//  * scheduler: every attended pair lies in a visited tile, every visited
//    tile holds an attended pair, FULL tiles hold only attended non-sink
//    pairs below n, the closed-form FULL run agrees with the per-tile test,
//    and the workgroup order is a permutation of (unit, query block).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "schedule.h"

extern "C" {
int swa_oracle_attended(long i, long j, long w, long g);
long swa_oracle_row_count(long i, long w, long g);
long swa_oracle_pair_count(long n, long w, long g);
int swa_oracle_mask(long n, long w, long g, unsigned char *out);
int swa_oracle_prefill(const double *q, const double *k, const double *v, long bh, long n, long d, long w, long g,
                       double scale, double beta, const long *rows, long nrows, double *o, double *lse,
                       int nthreads);
int swa_oracle_decode(const double *q, const long *p, const long *kpos, const double *k, const double *v, long units,
                      long nk, long d, long w, long g, double scale, double beta, double *o, double *lse,
                      int nthreads);
}

static int failures = 0;
#define CHECK(cond, ...)                                 \
    do {                                                 \
        if (!(cond)) {                                   \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);           \
            std::fprintf(stderr, "\n");                  \
            ++failures;                                  \
        }                                                \
    } while (0)

// deterministic inputs in [-1, 1) (a 64-bit LCG; any fixed values would do)
static std::vector<double> lcg_values(size_t count, unsigned long long seed) {
    std::vector<double> x(count);
    unsigned long long s = seed * 6364136223846793005ULL + 1442695040888963407ULL;
    for (auto &e : x) {
        s = s * 6364136223846793005ULL + 1442695040888963407ULL;
        e = (double)(s >> 11) / (double)(1ULL << 52) - 1.0;
    }
    return x;
}

static void oracle_counts() {
    CHECK(swa_oracle_pair_count(8, 3, 0) == 21, "8 tokens, window 3");
    CHECK(swa_oracle_pair_count(8, 8, 0) == 36 && swa_oracle_pair_count(8, 100, 0) == 36, "8 tokens causal");
    CHECK(swa_oracle_pair_count(6, 3, 0) == 15, "6 tokens, window 3");
    CHECK(swa_oracle_pair_count(8, 3, 1) == 26, "8 tokens, window 3, one sink");
    CHECK(swa_oracle_pair_count(256, 64, 0) == 14368, "256 tokens, window 64");
    for (long n = 1; n <= 60; ++n)
        for (long w = 1; w <= n; ++w)
            CHECK(swa_oracle_pair_count(n, w, 0) == n * w - w * (w - 1) / 2, "closed form n=%ld w=%ld", n, w);
    std::set<long> row7, row7a;
    for (long j = 0; j < 8; ++j) {
        if (swa_oracle_attended(7, j, 3, 0)) row7.insert(j);
        if (swa_oracle_attended(7, j, 3, 1)) row7a.insert(j);
    }
    CHECK((row7 == std::set<long>{5, 6, 7}), "row 7 window");
    CHECK((row7a == std::set<long>{0, 5, 6, 7}), "row 7 window and anchor");
    CHECK(!swa_oracle_attended(3, 4, 3, 1), "no future key");
    std::vector<unsigned char> m(40 * 40);
    CHECK(swa_oracle_mask(40, 7, 3, m.data()) == 0, "mask");
    long ones = 0;
    for (unsigned char c : m) ones += c;
    CHECK(ones == swa_oracle_pair_count(40, 7, 3), "mask ones");
}

static void oracle_values() {
    const long n = 37, d = 8, bh = 2;
    const double scale = 1.0 / std::sqrt((double)d);
    auto q = lcg_values(bh * n * d, 1), k = lcg_values(bh * n * d, 2), v = lcg_values(bh * n * d, 3);
    std::vector<double> o(bh * n * d), lse(bh * n), o2(bh * n * d);
    // window >= n: plain causal softmax attention, written out
    CHECK(swa_oracle_prefill(q.data(), k.data(), v.data(), bh, n, d, n + 3, 0, scale, 0.0, nullptr, 0, o.data(),
                             lse.data(), 1) == 0, "prefill");
    double worst = 0.0;
    for (long b = 0; b < bh; ++b)
        for (long i = 0; i < n; ++i) {
            const double *qi = &q[(b * n + i) * d];
            std::vector<double> s(i + 1);
            double mx = -INFINITY;
            for (long j = 0; j <= i; ++j) {
                double t = 0.0;
                for (long c = 0; c < d; ++c) t += qi[c] * k[(b * n + j) * d + c];
                s[j] = t * scale;
                mx = std::fmax(mx, s[j]);
            }
            double l = 0.0;
            for (long j = 0; j <= i; ++j) l += std::exp(s[j] - mx);
            for (long c = 0; c < d; ++c) {
                double acc = 0.0;
                for (long j = 0; j <= i; ++j) acc += std::exp(s[j] - mx) * v[(b * n + j) * d + c];
                worst = std::fmax(worst, std::fabs(acc / l - o[(b * n + i) * d + c]));
            }
            worst = std::fmax(worst, std::fabs(mx + std::log(l) - lse[b * n + i]));
        }
    CHECK(worst < 1e-12, "causal equivalence %.3g", worst);
    // window of 1, no sinks: o = v exactly
    CHECK(swa_oracle_prefill(q.data(), k.data(), v.data(), bh, n, d, 1, 0, scale, 0.0, nullptr, 0, o.data(), nullptr,
                             1) == 0, "prefill w=1");
    for (size_t e = 0; e < o.size(); ++e) CHECK(o[e] == v[e], "w=1 gives v at %zu", e);
    // zero queries: weights e^{beta [j < g]} over A_i
    const long w = 5, g = 3;
    const double beta = 1.25;
    std::vector<double> qz(bh * n * d, 0.0);
    CHECK(swa_oracle_prefill(qz.data(), k.data(), v.data(), bh, n, d, w, g, scale, beta, nullptr, 0, o.data(),
                             nullptr, 1) == 0, "prefill q=0");
    worst = 0.0;
    for (long b = 0; b < bh; ++b)
        for (long i = 0; i < n; ++i)
            for (long c = 0; c < d; ++c) {
                double num = 0.0, den = 0.0;
                for (long j = 0; j <= i; ++j) {
                    if (!(j >= i - w + 1 || j < g)) continue;
                    const double wt = std::exp(j < g ? beta : 0.0);
                    num += wt * v[(b * n + j) * d + c];
                    den += wt;
                }
                worst = std::fmax(worst, std::fabs(num / den - o[(b * n + i) * d + c]));
            }
    CHECK(worst < 1e-12, "zero-query closed form %.3g", worst);
    // decode over the logical sequence equals the prefill row (one unit per row)
    CHECK(swa_oracle_prefill(q.data(), k.data(), v.data(), 1, n, d, w, g, scale, beta, nullptr, 0, o.data(),
                             lse.data(), 1) == 0, "prefill for decode");
    const long nk = n;
    std::vector<long> p(n), kpos(n * nk);
    std::vector<double> qd(n * d), kd(n * nk * d), vd(n * nk * d), od(n * d), ld(n);
    for (long u = 0; u < n; ++u) {
        p[u] = u;
        for (long c = 0; c < d; ++c) qd[u * d + c] = q[u * d + c];
        for (long t = 0; t < nk; ++t) {
            // rows in reverse order, the ones past the query marked as padding
            const long j = nk - 1 - t;
            kpos[u * nk + t] = (j <= u) ? j : -1;
            for (long c = 0; c < d; ++c) {
                kd[(u * nk + t) * d + c] = k[j * d + c];
                vd[(u * nk + t) * d + c] = v[j * d + c];
            }
        }
    }
    CHECK(swa_oracle_decode(qd.data(), p.data(), kpos.data(), kd.data(), vd.data(), n, nk, d, w, g, scale, beta,
                            od.data(), ld.data(), 1) == 0, "decode");
    worst = 0.0;
    for (long e = 0; e < n * d; ++e) worst = std::fmax(worst, std::fabs(od[e] - o[e]));
    for (long u = 0; u < n; ++u) worst = std::fmax(worst, std::fabs(ld[u] - lse[u]));
    CHECK(worst < 1e-12, "decode = prefill row %.3g", worst);
    // a missing attended row is refused
    kpos[(n - 1) * nk + 0] = -1;  // drop key n-1 from the last unit
    CHECK(swa_oracle_decode(qd.data(), p.data(), kpos.data(), kd.data(), vd.data(), n, nk, d, w, g, scale, beta,
                            od.data(), ld.data(), 1) == -2, "incomplete key set refused");
}

static void schedule_shape(long n, long w, long g, int bq, int bk) {
    std::vector<unsigned char> mask(n * n);
    swa_oracle_mask(n, w, g, mask.data());
    std::vector<unsigned char> covered(n * n, 0);
    const int nqb = (int)((n + bq - 1) / bq);
    for (int qb = 0; qb < nqb; ++qb) {
        const int q0 = qb * bq, q1 = (int)std::min<long>(n, (long)(qb + 1) * bq) - 1;
        const swa::BandRange r = swa::band_range(q0, q1, (int)w, (int)g, bk);
        int t_lo, t_hi;
        swa::full_range(r, q0, q1, (int)n, (int)w, (int)g, bk, &t_lo, &t_hi);
        int prev = -1;
        for (int t = 0; t < r.count(); ++t) {
            const int kb = r.block(t);
            CHECK(kb > prev, "key blocks ascending (n=%ld w=%ld g=%ld qb=%d)", n, w, g, qb);
            prev = kb;
            const int k0 = kb * bk, k1 = kb * bk + bk - 1;
            bool any = false, all = true, sink = false;
            for (int i = q0; i <= q1; ++i)
                for (int j = k0; j <= k1; ++j) {
                    if (j >= n) {
                        all = false;
                        continue;
                    }
                    const bool a = mask[i * n + j] != 0;
                    any = any || a;
                    all = all && a;
                    sink = sink || (j < g);
                    covered[i * n + j] = 1;
                }
            CHECK(any, "tile (%d,%d) holds an attended pair (n=%ld w=%ld g=%ld)", qb, kb, n, w, g);
            const bool full = swa::tile_full(q0, q1, k0, k1, (int)n, (int)w, (int)g);
            CHECK(full == (all && !sink), "FULL test of tile (%d,%d) (n=%ld w=%ld g=%ld)", qb, kb, n, w, g);
            CHECK(full == (t >= t_lo && t < t_hi), "closed-form FULL run (n=%ld w=%ld g=%ld)", n, w, g);
        }
    }
    for (long e = 0; e < n * n; ++e)
        CHECK(!mask[e] || covered[e], "pair (%ld,%ld) in a visited tile (n=%ld w=%ld g=%ld)", e / n, e % n, n, w, g);
}

static void schedule_checks() {
    const long shapes[][3] = {{8, 3, 0},     {8, 3, 1},     {257, 1, 0},   {257, 63, 0}, {257, 64, 4},
                              {257, 65, 0},  {300, 300, 0}, {300, 1000, 2}, {500, 127, 65}, {500, 129, 130},
                              {377, 300, 4}, {64, 64, 64},  {129, 5, 200}};
    const int tiles[][2] = {{128, 64}, {64, 64}, {32, 32}, {128, 128}, {16, 48}, {256, 32}};
    for (const auto &s : shapes)
        for (const auto &t : tiles) schedule_shape(s[0], s[1], s[2], t[0], t[1]);
    const int orders[][3] = {{1, 1, 1}, {1, 7, 1}, {3, 5, 1}, {32, 128, 1}, {5, 13, 1}, {2, 3, 1}, {16, 1024, 1},
                             {32, 128, 4}, {8, 5, 8}, {6, 7, 3}, {4, 3, 2}};
    for (const auto &o : orders) {
        const int units = o[0], nqb = o[1], group = o[2], total = units * nqb;
        std::vector<unsigned char> seen(total, 0);
        for (int bid = 0; bid < total; ++bid) {
            int u, qb;
            swa::workgroup_order(bid, total, nqb, group, &u, &qb);
            CHECK(u >= 0 && u < units && qb >= 0 && qb < nqb, "order in range");
            if (u >= 0 && u < units && qb >= 0 && qb < nqb) {
                CHECK(!seen[u * nqb + qb], "order visits (%d,%d) once", u, qb);
                seen[u * nqb + qb] = 1;
            }
        }
    }
}

int main() {
    oracle_counts();
    oracle_values();
    schedule_checks();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("sanitized host checks: ok\n");
    return 0;
}
