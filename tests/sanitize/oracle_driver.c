/* Runs every entry point of the fp64 oracle on tiny seeded inputs (several
 * shapes, with and without the forget gate, decode with and without a new
 * token), built with AddressSanitizer and UndefinedBehaviorSanitizer; checks
 * that the results are finite.  Its numbers are pinned elsewhere. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fwd(const double *, const double *, const double *, const double *, const double *, const double *, int,
               int, int, double, const int64_t *, int64_t, double *, double *, int);
void oracle_scores_head(const double *, const double *, const double *, const double *, const double *, int, int,
                        double, double *);
void oracle_transport(const double *, const double *, const double *, int, int, int, double *);
int oracle_decode(double *, double *, double *, int64_t, int64_t, const double *, const double *, const double *,
                  const double *, const double *, const double *, int, int, double, double *, double *, int);
int oracle_decode_cache(const double *, const double *, const double *, const double *, int, int, int, double *,
                        double *);
int oracle_produce(const double *, const double *, const double *, double, int, int, int, int, double *, double *);
int oracle_bwd(const double *, const double *, const double *, const double *, const double *, const double *,
               const double *, const double *, int, int, int, double, double *, double *, double *, double *,
               double *, double *, double *, double *, int);

static uint64_t st = 12345;
static double rnd(void) { /* uniform in (-1, 1), xorshift64 */
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return ((double)(st >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}
static double *arr(size_t n, double lo, double hi) {
    double *a = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * 0.5 * (rnd() + 1.0);
    return a;
}
static int bad = 0;
static void finite(const char *what, const double *a, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) { printf("FAIL %s: non-finite at %zu\n", what, i); ++bad; return; }
}

int main(void) {
    const int shapes[][3] = {{1, 1, 4}, {2, 2, 8}, {1, 5, 8}, {2, 64, 16}, {1, 70, 64}};
    for (unsigned s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const int G = shapes[s][0], L = shapes[s][1], d = shapes[s][2];
        const size_t n = (size_t)G * L * d, t = (size_t)G * L;
        double *q = arr(n, -1, 1), *k = arr(n, -1, 1), *v = arr(n, -1, 1), *w = arr(n, -1, 1);
        double *beta = arr(t, 0, 2), *logf = arr(t, -0.2, 0), *out = arr(n, 0, 0), *lse = arr(t, 0, 0);
        for (int gate = 0; gate < 2; ++gate) {
            if (oracle_fwd(q, k, v, w, beta, gate ? logf : NULL, G, L, d, 0.3, NULL, 0, out, lse, 2)) ++bad;
            finite("fwd out", out, n);
            finite("fwd lse", lse, t);
            int64_t rows[4] = {0, L - 1, G - 1, 0};
            double ro[2 * 64], rl[2];
            if (oracle_fwd(q, k, v, w, beta, gate ? logf : NULL, G, L, d, 0.3, rows, 2, ro, rl, 1)) ++bad;
            finite("fwd rows", ro, 2 * (size_t)d);
            double *S = arr((size_t)L * L, 0, 0);
            oracle_scores_head(q, k, w, beta, gate ? logf : NULL, L, d, 0.3, S);
            free(S);
            double *dout = arr(n, -1, 1), *dlse = arr(t, -1, 1), *g[8];
            for (int u = 0; u < 4; ++u) g[u] = arr(n, 0, 0);
            g[4] = arr(t, 0, 0); g[5] = arr(t, 0, 0); g[6] = arr(n, 0, 0); g[7] = arr(t, 0, 0);
            if (oracle_bwd(q, k, v, w, beta, gate ? logf : NULL, dout, gate ? dlse : NULL, G, L, d, 0.3, g[0], g[1],
                           g[2], g[3], g[4], gate ? g[5] : NULL, g[6], g[7], 3)) ++bad;
            for (int u = 0; u < 4; ++u) finite("bwd grads", g[u], n);
            finite("bwd dbeta", g[4], t);
            for (int u = 0; u < 8; ++u) free(g[u]);
            free(dout); free(dlse);
            double *kc = arr(n, 0, 0), *fc = arr(t, 0, 0);
            if (oracle_decode_cache(k, w, beta, gate ? logf : NULL, G, L, d, kc, gate ? fc : NULL)) ++bad;
            finite("decode cache", kc, n);
            free(kc); free(fc);
        }
        double x[64], o[64];
        for (int c = 0; c < d; ++c) x[c] = rnd();
        oracle_transport(x, w, beta, d, 0, L - 1, o);
        finite("transport", o, (size_t)d);
        /* decode: cache of L rows plus room for one more */
        const int64_t cap = L + 1;
        double *kc = arr((size_t)G * cap * d, -1, 1), *vc = arr((size_t)G * cap * d, -1, 1), *fc = arr((size_t)G * cap, -1, 0);
        double *qd = arr((size_t)G * d, -1, 1), *wd = arr((size_t)G * d, -1, 1), *bd = arr(G, 0, 2), *lf = arr(G, -0.2, 0);
        double *kn = arr((size_t)G * d, -1, 1), *vn = arr((size_t)G * d, -1, 1), *od = arr((size_t)G * d, 0, 0), *ld = arr(G, 0, 0);
        for (int app = 0; app < 2; ++app)
            for (int gate = 0; gate < 2; ++gate) {
                if (oracle_decode(kc, vc, gate ? fc : NULL, L, cap, qd, wd, bd, gate ? lf : NULL, app ? kn : NULL,
                                  app ? vn : NULL, G, d, 0.3, od, ld, 2)) ++bad;
                finite("decode out", od, (size_t)G * d);
            }
        double *cw = arr((size_t)L * d * 3, -1, 1), *z = arr(t, -2, 2), *wp = arr(n, 0, 0), *bp = arr(t, 0, 0);
        if (oracle_produce(v, cw, z, s % 2 ? 1.9 : 0.0, G, 1, L, d, wp, bp)) ++bad;
        finite("produce w", wp, n);
        free(cw); free(z); free(wp); free(bp);
        free(kc); free(vc); free(fc); free(qd); free(wd); free(bd); free(lf); free(kn); free(vn); free(od); free(ld);
        free(q); free(k); free(v); free(w); free(beta); free(logf); free(out); free(lse);
    }
    printf("%s: %d failures\n", bad ? "FAILED" : "oracle ok", bad);
    return bad ? 1 : 0;
}
