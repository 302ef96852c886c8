/*
 * path_oracle.c -- plain, slow, fp64 CPU oracle for PaTH attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with
 * the HIP library.
 *
 * Sources (cited by page title and section):
 *   [TS]  "技術要約: PaTH Attention" (gist.science, Japanese technical summary
 *         of arXiv 2505.16381), section 2 "手法" (attention-logit formula,
 *         transition matrix H_s, range of beta) and section 3 "効率的な学習と推論"
 *         (inference: historical keys are updated in place with the newest
 *         transition matrix).
 *   [IPX] "거리에서 경로로, PaTH Attention" (iplexlaw.co.kr blog), section 3
 *         (score k_j^T (H_{j+1} ... H_i) q_i, then softmax and a weighted sum of
 *         values) and section 4 (PaTH-FoX adds a forget gate).
 *
 * What is computed (the definition, written out, no blocking or reordering):
 *   H_s = I - beta_s w_s w_s^T                                  [TS s.2]
 *   s_ij = scale * k_j^T (H_{j+1} H_{j+2} ... H_i) q_i,  j <= i  [TS s.2, IPX s.3]
 *          (+ sum_{s=j+1..i} log f_s  when a log-forget gate is given)
 *   p_ij = softmax over j <= i of s_ij,  o_i = sum_j p_ij v_j    [IPX s.3-4]
 * The pages print the logit without a 1/sqrt(d) factor and give no formula
 * for the forget gate; the readings taken are: `scale` multiplies the product
 * term only, and the forget-gate bias is the sum of log f_s over the path
 * s = j+1..i, added unscaled (zero on the diagonal).
 *
 * Evaluation order: for a query row i the vector u = H_{j+1} ... H_i q_i is
 * built by applying the H's one at a time, starting from u = q_i (empty
 * product, j = i) and stepping j downward: u <- H_{j+1} u.  Applying H to a
 * vector is u - beta (w . u) w, which is H u exactly.  Cost O(i d) per row.
 *
 * Decode [TS s.3]: the newest transition H_t is applied to every cached key
 * in place (k_j <- H_t k_j), after which a single query attends to the cache.
 * Since every H is symmetric, a cache row that holds H_t ... H_{j+1} k_j gives
 * (H_t ... H_{j+1} k_j)^T q_t = k_j^T (H_{j+1} ... H_t) q_t, the forward logit.
 * A new key/value (if given) enters after the update, untransformed, because
 * the logit of j = t has the empty product.
 *
 * Decode with the forget gate: the bias of row j at step t is the path sum
 * sum_{s=j+1..t} log f_s = c_t - c_j with c_j = sum_{s<=j} log f_s, so a
 * cache of c_j per row (and the newest c_t = c_{t-1} + log f_t) is enough.
 *
 * Decode cache after a prefix of L tokens [TS s.3]: if tokens 0 .. L-1 had
 * been fed one decode step at a time, cache row j would have been updated by
 * steps j+1, ..., L-1 in that order, so it holds H_{L-1} ... H_{j+1} k_j
 * (H_{j+1} acts first; row L-1 is k_{L-1} itself).
 *
 * Producer of w and beta [IPX s.3; TS s.2; "PaTH Attention" Chinese summary,
 * method paragraph]: w comes out of a low-dimensional linear projection, a
 * short convolution of width 3 and an L2 normalisation; beta = 2 sigmoid(u^T
 * x + b), so it lies in (0, 2).  The projections are ordinary matrix products
 * outside this function, which takes their outputs: the pre-convolution rows
 * x_t (wraw) and the pre-sigmoid values z_t.  Readings: the convolution is
 * causal and per channel (depthwise), tap tau = 0, 1, 2 multiplying x_{t-2+tau}
 * (zero before the first token), no bias, no activation; the normalisation is
 * y / max(||y||, 1e-12); a positive beta_clip caps beta (the pages ask for
 * clipping near 2 in bf16 without a value).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* u <- H u with H = I - beta w w^T (one transition matrix applied to a vector). */
static void apply_h(double *u, const double *w, double beta, int d) {
    double wu = 0.0;
    for (int c = 0; c < d; ++c) wu += w[c] * u[c];
    for (int c = 0; c < d; ++c) u[c] -= beta * wu * w[c];
}

/*
 * out = H_lo H_{lo+1} ... H_hi x  (product in increasing index order, applied
 * to x, so H_hi acts first).  lo > hi means the empty product (out = x).
 * w is [n, d] row-major, beta is [n].
 */
void oracle_transport(const double *x, const double *w, const double *beta, int d, int lo, int hi,
                      double *out) {
    memcpy(out, x, sizeof(double) * (size_t)d);
    for (int s = hi; s >= lo; --s) apply_h(out, w + (size_t)s * d, beta[s], d);
}

/*
 * All logits of one head: S[i*L + j] = s_ij for j <= i, -INFINITY for j > i.
 * logf may be NULL (plain PaTH).
 */
void oracle_scores_head(const double *q, const double *k, const double *w, const double *beta,
                        const double *logf, int L, int d, double scale, double *S) {
    double *u = (double *)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
    for (int i = 0; i < L; ++i) {
        memcpy(u, q + (size_t)i * d, sizeof(double) * (size_t)d);
        double bias = 0.0;
        for (int j = i; j >= 0; --j) {
            if (j < i) {
                apply_h(u, w + (size_t)(j + 1) * d, beta[j + 1], d);
                if (logf) bias += logf[j + 1];
            }
            double kt = 0.0;
            for (int c = 0; c < d; ++c) kt += k[(size_t)j * d + c] * u[c];
            S[(size_t)i * L + j] = scale * kt + bias;
        }
        for (int j = i + 1; j < L; ++j) S[(size_t)i * L + j] = -INFINITY;
    }
    free(u);
}

/*
 * One output row of one head: o_i and lse_i = log sum_j exp(s_ij).
 * sbuf is caller scratch of length >= i+1, u of length d.
 */
static void fwd_row(const double *q, const double *k, const double *v, const double *w,
                    const double *beta, const double *logf, int d, double scale, int i,
                    double *sbuf, double *u, double *o, double *lse) {
    memcpy(u, q + (size_t)i * d, sizeof(double) * (size_t)d);
    double bias = 0.0;
    double m = -INFINITY;
    for (int j = i; j >= 0; --j) {
        if (j < i) {
            apply_h(u, w + (size_t)(j + 1) * d, beta[j + 1], d);
            if (logf) bias += logf[j + 1];
        }
        double kt = 0.0;
        for (int c = 0; c < d; ++c) kt += k[(size_t)j * d + c] * u[c];
        sbuf[j] = scale * kt + bias;
        if (sbuf[j] > m) m = sbuf[j];
    }
    double z = 0.0;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int j = 0; j <= i; ++j) {
        double p = exp(sbuf[j] - m);
        z += p;
        for (int c = 0; c < d; ++c) o[c] += p * v[(size_t)j * d + c];
    }
    for (int c = 0; c < d; ++c) o[c] /= z;
    *lse = m + log(z);
}

typedef struct {
    const double *q, *k, *v, *w, *beta, *logf;
    int G, L, d;
    double scale;
    const int64_t *rows; /* pairs (g, i); NULL = every row of every head */
    int64_t nrows;
    double *out, *lse;
    int64_t next; /* work counter, protected by mu */
    pthread_mutex_t mu;
} fwd_job_t;

static void *fwd_worker(void *arg) {
    fwd_job_t *jb = (fwd_job_t *)arg;
    int L = jb->L, d = jb->d;
    double *sbuf = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double *u = (double *)malloc(sizeof(double) * (size_t)d);
    int64_t total = jb->rows ? jb->nrows : (int64_t)jb->G * L;
    for (;;) {
        int64_t t0;
        pthread_mutex_lock(&jb->mu);
        t0 = jb->next;
        jb->next += 16;
        pthread_mutex_unlock(&jb->mu);
        if (t0 >= total) break;
        int64_t t1 = t0 + 16 < total ? t0 + 16 : total;
        for (int64_t t = t0; t < t1; ++t) {
            int64_t g, i;
            if (jb->rows) {
                g = jb->rows[2 * t];
                i = jb->rows[2 * t + 1];
            } else {
                g = t / L;
                i = t % L;
            }
            size_t hd = (size_t)g * L * d;
            const double *lf = jb->logf ? jb->logf + (size_t)g * L : NULL;
            fwd_row(jb->q + hd, jb->k + hd, jb->v + hd, jb->w + hd, jb->beta + (size_t)g * L, lf, d,
                    jb->scale, (int)i, sbuf, u, jb->out + (size_t)t * d, jb->lse + t);
        }
    }
    free(sbuf);
    free(u);
    return NULL;
}

/*
 * Forward over G independent heads, each [L, d] row-major (beta, logf: [L]).
 * rows == NULL: every row; out is [G, L, d], lse [G, L].
 * rows != NULL: nrows pairs (g, i); out is [nrows, d], lse [nrows].
 * Returns 0 on success, -1 on bad arguments.
 */
int oracle_fwd(const double *q, const double *k, const double *v, const double *w, const double *beta,
               const double *logf, int G, int L, int d, double scale, const int64_t *rows, int64_t nrows,
               double *out, double *lse, int nthreads) {
    if (G < 0 || L < 0 || d < 1 || nthreads < 1) return -1;
    if (rows) {
        for (int64_t t = 0; t < nrows; ++t)
            if (rows[2 * t] < 0 || rows[2 * t] >= G || rows[2 * t + 1] < 0 || rows[2 * t + 1] >= L) return -1;
    }
    fwd_job_t jb;
    jb.q = q; jb.k = k; jb.v = v; jb.w = w; jb.beta = beta; jb.logf = logf;
    jb.G = G; jb.L = L; jb.d = d; jb.scale = scale;
    jb.rows = rows; jb.nrows = nrows; jb.out = out; jb.lse = lse; jb.next = 0;
    pthread_mutex_init(&jb.mu, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, fwd_worker, &jb);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&jb.mu);
    return 0;
}

/*
 * One decode step for one head [TS s.3].
 *   kc: [n (+1 if knew), d] cache rows, updated in place: k_j <- H_t k_j for j < n.
 *   vc: [n (+1), d].  If knew/vnew are non-NULL they are written to row n after
 *   the update and the query attends to n+1 rows; otherwise to n rows.
 *   q, w: [d]; beta: scalar.  out: [d]; lse: scalar.
 */
static void decode_head(double *kc, double *vc, double *fc, int64_t n, const double *q, const double *w,
                        double beta, const double *logf, const double *knew, const double *vnew, int d,
                        double scale, double *out, double *lse) {
    for (int64_t j = 0; j < n; ++j) apply_h(kc + (size_t)j * d, w, beta, d);
    /* forget gate: c_t of the current token; row j gets c_t - c_j */
    const double ct = logf ? (n > 0 ? fc[n - 1] : 0.0) + *logf : 0.0;
    int64_t nt = n;
    if (knew && vnew) {
        memcpy(kc + (size_t)n * d, knew, sizeof(double) * (size_t)d);
        memcpy(vc + (size_t)n * d, vnew, sizeof(double) * (size_t)d);
        if (logf) fc[n] = ct;
        nt = n + 1;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < nt; ++j) {
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += kc[(size_t)j * d + c] * q[c];
        s *= scale;
        if (logf) s += ct - fc[j];
        if (s > m) m = s;
    }
    double z = 0.0;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int64_t j = 0; j < nt; ++j) {
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += kc[(size_t)j * d + c] * q[c];
        double p = exp(scale * s + (logf ? ct - fc[j] : 0.0) - m);
        z += p;
        for (int c = 0; c < d; ++c) out[c] += p * vc[(size_t)j * d + c];
    }
    for (int c = 0; c < d; ++c) out[c] /= z;
    *lse = m + log(z);
}

typedef struct {
    double *kc, *vc, *fc;
    int64_t n, rowcap;
    const double *q, *w, *beta, *logf, *knew, *vnew;
    int G, d;
    double scale;
    double *out, *lse;
    int next;
    pthread_mutex_t mu;
} dec_job_t;

static void *dec_worker(void *arg) {
    dec_job_t *jb = (dec_job_t *)arg;
    for (;;) {
        int g;
        pthread_mutex_lock(&jb->mu);
        g = jb->next++;
        pthread_mutex_unlock(&jb->mu);
        if (g >= jb->G) break;
        size_t base = (size_t)g * (size_t)jb->rowcap * jb->d;
        decode_head(jb->kc + base, jb->vc + base, jb->fc ? jb->fc + (size_t)g * (size_t)jb->rowcap : NULL, jb->n,
                    jb->q + (size_t)g * jb->d, jb->w + (size_t)g * jb->d, jb->beta[g], jb->logf ? jb->logf + g : NULL,
                    jb->knew ? jb->knew + (size_t)g * jb->d : NULL,
                    jb->vnew ? jb->vnew + (size_t)g * jb->d : NULL, jb->d, jb->scale,
                    jb->out + (size_t)g * jb->d, jb->lse + g);
    }
    return NULL;
}

/*
 * Decode step over G heads.  kc, vc: [G, rowcap, d]; rows [0, n) are the cache
 * (kc updated in place); with knew/vnew ([G, d]) rowcap must be >= n+1.
 * q, w: [G, d]; beta: [G]; out: [G, d]; lse: [G].
 * Forget gate (both or neither): logf [G] = log f_t, fc [G, rowcap] = c_j per
 * cached row (c_n is written when knew/vnew are given).  Returns 0 or -1.
 */
int oracle_decode(double *kc, double *vc, double *fc, int64_t n, int64_t rowcap, const double *q, const double *w,
                  const double *beta, const double *logf, const double *knew, const double *vnew, int G, int d,
                  double scale, double *out, double *lse, int nthreads) {
    if (G < 0 || d < 1 || n < 0 || nthreads < 1) return -1;
    if ((knew == NULL) != (vnew == NULL)) return -1;
    if ((logf == NULL) != (fc == NULL)) return -1;
    if (rowcap < n + (knew ? 1 : 0)) return -1;
    if (n + (knew ? 1 : 0) < 1) return -1;
    dec_job_t jb;
    jb.kc = kc; jb.vc = vc; jb.fc = fc; jb.n = n; jb.rowcap = rowcap;
    jb.q = q; jb.w = w; jb.beta = beta; jb.logf = logf; jb.knew = knew; jb.vnew = vnew;
    jb.G = G; jb.d = d; jb.scale = scale; jb.out = out; jb.lse = lse; jb.next = 0;
    pthread_mutex_init(&jb.mu, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, dec_worker, &jb);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&jb.mu);
    return 0;
}

/*
 * Decode cache of G heads after a prefix of L tokens: out[g][j] =
 * H_{L-1} ... H_{j+1} k_j, applying H_{j+1} first and H_{L-1} last (the order
 * of the in-place decode updates).  k, w: [G, L, d]; beta: [G, L];
 * out: [G, L, d].  With the forget gate, logf [G, L] gives the gate cache
 * fc[g][j] = sum_{s<=j} log f_s (fc: [G, L]).  Returns 0 or -1.
 */
int oracle_decode_cache(const double *k, const double *w, const double *beta, const double *logf, int G, int L,
                        int d, double *out, double *fc) {
    if (G < 0 || L < 0 || d < 1 || ((logf == NULL) != (fc == NULL))) return -1;
    if (logf) {
        for (int g = 0; g < G; ++g) {
            double c = 0.0;
            for (int j = 0; j < L; ++j) {
                c += logf[(size_t)g * L + j];
                fc[(size_t)g * L + j] = c;
            }
        }
    }
    for (int g = 0; g < G; ++g) {
        const double *kg = k + (size_t)g * L * d, *wg = w + (size_t)g * L * d, *bg = beta + (size_t)g * L;
        double *og = out + (size_t)g * L * d;
        for (int j = 0; j < L; ++j) {
            double *u = og + (size_t)j * d;
            memcpy(u, kg + (size_t)j * d, sizeof(double) * (size_t)d);
            for (int s = j + 1; s < L; ++s) apply_h(u, wg + (size_t)s * d, bg[s], d);
        }
    }
    return 0;
}

/*
 * Producer of w and beta (see the header): for every head g (conv weights of
 * head g % H), token t and channel c
 *   y_t[c] = sum_{tau=0..2} cw[(g % H)][c][tau] * x_{t-2+tau}[c]   (x_{<0} = 0)
 *   w_t = y_t / max(||y_t||, 1e-12),  beta_t = 2 / (1 + exp(-z_t)), capped at
 *   beta_clip when beta_clip > 0.
 * wraw: [G, L, d], cw: [H, d, 3], z: [G, L]; out w: [G, L, d], beta: [G, L].
 * Returns 0 or -1.
 */
int oracle_produce(const double *wraw, const double *cw, const double *z, double beta_clip, int G, int H, int L,
                   int d, double *w, double *beta) {
    if (G < 0 || H < 1 || L < 0 || d < 1 || G % H != 0) return -1;
    for (int g = 0; g < G; ++g) {
        const double *x = wraw + (size_t)g * L * d, *cwh = cw + (size_t)(g % H) * d * 3;
        for (int t = 0; t < L; ++t) {
            double *y = w + ((size_t)g * L + t) * d;
            double nn = 0.0;
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int tau = 0; tau < 3; ++tau) {
                    const int src = t - 2 + tau;
                    if (src >= 0) acc += cwh[(size_t)c * 3 + tau] * x[(size_t)src * d + c];
                }
                y[c] = acc;
                nn += acc * acc;
            }
            const double nrm = fmax(sqrt(nn), 1e-12);
            for (int c = 0; c < d; ++c) y[c] /= nrm;
            double b = 2.0 / (1.0 + exp(-z[(size_t)g * L + t]));
            if (beta_clip > 0.0 && b > beta_clip) b = beta_clip;
            beta[(size_t)g * L + t] = b;
        }
    }
    return 0;
}
