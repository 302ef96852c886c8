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
 *
 * Backward (oracle_bwd, at the end of this file): the gradient of the forward
 * by reverse mode of the same definition, row by row; see the comment there.
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

/*
 * Backward pass: the exact gradient of the forward above, by reverse mode of
 * the definition, one query row at a time.  The pages present the blockwise
 * algorithm as what makes PaTH trainable ([TS s.3]) but print no gradient
 * formulas, so this is the chain rule applied to the definition of [TS s.2]
 * and [IPX s.3-4], with nothing reordered beyond what the chain rule states.
 *
 * Loss whose gradient is taken: sum_i do_i . o_i + sum_i dlse_i lse_i, where
 * o and lse are this file's forward outputs (dlse may be NULL, i.e. zero).
 *
 * For row i, with u_j = H_{j+1} ... H_i q_i (u_i = q_i, u_{j-1} = H_j u_j):
 *   s_ij = scale k_j . u_j + (c_i - c_j),  P_ij = softmax_j,  o_i = sum_j P_ij v_j
 *   dP_ij = do_i . v_j;  dS_ij = P_ij (dP_ij - do_i . o_i + dlse_i)
 *   dv_j += P_ij do_i;   dk_j += scale dS_ij u_j
 * The adjoint lam_j of u_j collects scale dS_ij k_j from the logit of key j
 * and H_j lam_{j-1} from u_{j-1} = H_j u_j (H is symmetric); the same step
 * gives dH_j = lam_{j-1} u_j^T, whose projections on H_j = I - beta_j w_j w_j^T are
 *   dbeta_j -= (w_j . lam_{j-1}) (w_j . u_j)
 *   dw_j    -= beta_j ((w_j . u_j) lam_{j-1} + (w_j . lam_{j-1}) u_j).
 * Walking j = 0 .. i upward ends with dq_i = lam_i.  The gate bias c_i - c_j
 * is the sum of log f_t over t = j+1 .. i, so dlogf_t += sum_{j<t} dS_ij for
 * every t <= i.
 */
static void bwd_row(const double *q, const double *k, const double *v, const double *w, const double *beta,
                    const double *logf, const double *dout, const double *dlse, int d, double scale, int i,
                    double *U, double *s, double *lam, double *dq, double *dk, double *dv, double *dw,
                    double *dbeta, double *dlogf, double *o, double *lse) {
    /* states u_j for j = i .. 0 and the logits */
    memcpy(U + (size_t)i * d, q + (size_t)i * d, sizeof(double) * (size_t)d);
    for (int j = i - 1; j >= 0; --j) {
        memcpy(U + (size_t)j * d, U + (size_t)(j + 1) * d, sizeof(double) * (size_t)d);
        apply_h(U + (size_t)j * d, w + (size_t)(j + 1) * d, beta[j + 1], d);
    }
    double bias = 0.0, m = -INFINITY;
    for (int j = i; j >= 0; --j) {
        if (j < i && logf) bias += logf[j + 1];
        double kt = 0.0;
        for (int c = 0; c < d; ++c) kt += k[(size_t)j * d + c] * U[(size_t)j * d + c];
        s[j] = scale * kt + bias;
        if (s[j] > m) m = s[j];
    }
    double z = 0.0;
    for (int j = 0; j <= i; ++j) z += exp(s[j] - m);
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int j = 0; j <= i; ++j) {
        s[j] = exp(s[j] - m) / z; /* s now holds P_ij */
        for (int c = 0; c < d; ++c) o[c] += s[j] * v[(size_t)j * d + c];
    }
    *lse = m + log(z);
    const double *doi = dout + (size_t)i * d;
    double D = 0.0;
    for (int c = 0; c < d; ++c) D += doi[c] * o[c];
    const double gl = dlse ? dlse[i] : 0.0;
    for (int j = 0; j <= i; ++j) {
        double dp = 0.0;
        for (int c = 0; c < d; ++c) dp += doi[c] * v[(size_t)j * d + c];
        const double P = s[j];
        for (int c = 0; c < d; ++c) dv[(size_t)j * d + c] += P * doi[c];
        s[j] = P * (dp - D + gl); /* s now holds dS_ij */
        for (int c = 0; c < d; ++c) dk[(size_t)j * d + c] += scale * s[j] * U[(size_t)j * d + c];
    }
    /* adjoints, j upward */
    for (int c = 0; c < d; ++c) lam[c] = scale * s[0] * k[c];
    for (int j = 1; j <= i; ++j) {
        const double *wj = w + (size_t)j * d, *uj = U + (size_t)j * d;
        double a = 0.0, b = 0.0;
        for (int c = 0; c < d; ++c) {
            a += wj[c] * lam[c];
            b += wj[c] * uj[c];
        }
        dbeta[j] -= a * b;
        for (int c = 0; c < d; ++c) dw[(size_t)j * d + c] -= beta[j] * (b * lam[c] + a * uj[c]);
        for (int c = 0; c < d; ++c) lam[c] += -beta[j] * a * wj[c] + scale * s[j] * k[(size_t)j * d + c];
    }
    memcpy(dq, lam, sizeof(double) * (size_t)d);
    if (logf) {
        double acc = 0.0;
        for (int t = 1; t <= i; ++t) {
            acc += s[t - 1];
            dlogf[t] += acc;
        }
    }
}

typedef struct {
    const double *q, *k, *v, *w, *beta, *logf, *dout, *dlse;
    int L, d, nthreads, tid;
    double scale;
    double *dq, *acc; /* acc: this thread's [dk | dv | dw] (3 L d) then [dbeta | dlogf] (2 L) */
    double *o, *lse;
} bwd_job_t;

static void *bwd_worker(void *arg) {
    bwd_job_t *jb = (bwd_job_t *)arg;
    const int L = jb->L, d = jb->d;
    double *U = (double *)malloc(sizeof(double) * (size_t)L * d);
    double *s = (double *)malloc(sizeof(double) * (size_t)L);
    double *lam = (double *)malloc(sizeof(double) * (size_t)d);
    const size_t Ld = (size_t)L * d;
    for (int i = jb->tid; i < L; i += jb->nthreads)
        bwd_row(jb->q, jb->k, jb->v, jb->w, jb->beta, jb->logf, jb->dout, jb->dlse, d, jb->scale, i, U, s, lam,
                jb->dq + (size_t)i * d, jb->acc, jb->acc + Ld, jb->acc + 2 * Ld, jb->acc + 3 * Ld,
                jb->acc + 3 * Ld + L, jb->o + (size_t)i * d, jb->lse + i);
    free(U);
    free(s);
    free(lam);
    return NULL;
}

/*
 * Backward over G heads ([L, d] row-major each; beta, logf, dlse: [L]).
 * Inputs q, k, v, w, beta, logf (NULL = no gate), dout = dLoss/do [G, L, d],
 * dlse = dLoss/dlse [G, L] (NULL = 0).  Outputs dq, dk, dv, dw [G, L, d],
 * dbeta [G, L], dlogf [G, L] (only with logf), and the forward's o [G, L, d]
 * and lse [G, L].  Threads split the rows of a head; each keeps its own
 * key-side sums, added in thread order at the end (deterministic).
 * Returns 0 or -1.
 */
int oracle_bwd(const double *q, const double *k, const double *v, const double *w, const double *beta,
               const double *logf, const double *dout, const double *dlse, int G, int L, int d, double scale,
               double *dq, double *dk, double *dv, double *dw, double *dbeta, double *dlogf, double *o, double *lse,
               int nthreads) {
    if (G < 0 || L < 0 || d < 1 || nthreads < 1 || ((logf == NULL) != (dlogf == NULL))) return -1;
    if (nthreads > L) nthreads = L > 0 ? L : 1;
    const size_t Ld = (size_t)L * d, accn = 3 * Ld + 2 * (size_t)L;
    double *acc = (double *)malloc(sizeof(double) * accn * (size_t)nthreads);
    bwd_job_t *jobs = (bwd_job_t *)malloc(sizeof(bwd_job_t) * (size_t)nthreads);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int g = 0; g < G; ++g) {
        const size_t hd = (size_t)g * Ld, hl = (size_t)g * L;
        memset(acc, 0, sizeof(double) * accn * (size_t)nthreads);
        for (int t = 0; t < nthreads; ++t) {
            bwd_job_t *jb = &jobs[t];
            jb->q = q + hd; jb->k = k + hd; jb->v = v + hd; jb->w = w + hd; jb->beta = beta + hl;
            jb->logf = logf ? logf + hl : NULL; jb->dout = dout + hd; jb->dlse = dlse ? dlse + hl : NULL;
            jb->L = L; jb->d = d; jb->nthreads = nthreads; jb->tid = t; jb->scale = scale;
            jb->dq = dq + hd; jb->acc = acc + accn * (size_t)t; jb->o = o + hd; jb->lse = lse + hl;
            pthread_create(&th[t], NULL, bwd_worker, jb);
        }
        for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
        for (size_t e = 0; e < Ld; ++e) {
            double a = 0.0, b = 0.0, c = 0.0;
            for (int t = 0; t < nthreads; ++t) {
                a += acc[accn * (size_t)t + e];
                b += acc[accn * (size_t)t + Ld + e];
                c += acc[accn * (size_t)t + 2 * Ld + e];
            }
            dk[hd + e] = a;
            dv[hd + e] = b;
            dw[hd + e] = c;
        }
        for (int j = 0; j < L; ++j) {
            double a = 0.0, b = 0.0;
            for (int t = 0; t < nthreads; ++t) {
                a += acc[accn * (size_t)t + 3 * Ld + j];
                b += acc[accn * (size_t)t + 3 * Ld + L + j];
            }
            dbeta[hl + j] = a;
            if (dlogf) dlogf[hl + j] = b;
        }
    }
    free(acc);
    free(jobs);
    free(th);
    return 0;
}
