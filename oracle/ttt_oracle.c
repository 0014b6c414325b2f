/*
 * Plain sequential CPU oracle for the TTT-layer forward (test infrastructure).
 *
 * This file is the reference the HIP path is checked against.  It is test
 * infrastructure only: tests, the smoke check and the CPU-baseline leg of the
 * benchmark may call it; the library path never does.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Arithmetic: fp64 throughout, token by token, with the gradient of each
 * token's loss written out explicitly.  No blocking, no dual form, no reordering
 * beyond what the definitions below state.  Parallelism: independent
 * (batch, head) pairs may run on separate OpenMP threads; each pair's loop is
 * sequential.
 *
 * Sources (web pages; sections as titled on the pages):
 *  [TTT]  "Test-Time Training (TTT)" summary of *Learning to (Learn at Test
 *         Time): RNNs with Expressive Hidden States*:
 *           - "Mathematical definition / TTT definition": fast weight W_t,
 *             update W_t = W_{t-1} - eta_t * grad L, query y_t = f(q_t, W_t);
 *           - "How TTT generalises linear attention", example 1 (inner-product
 *             loss L = -(k W) . v, gradient -k^T v) and example 2 (MSE loss
 *             L = 1/2 ||k W - v||^2, gradient k^T (k W - v));
 *           - "TTT variants / TTT-Linear": f(x, W) = x W, a d x d state;
 *           - "Parallelisation: mini-batch gradient descent": within a chunk
 *             every token's gradient is taken at the chunk-start state and the
 *             chunk's gradients are summed.
 *  [LaCT] "LaCT: Test-Time Training Done Right" analysis:
 *           - section 3.2: SwiGLU fast-weight MLP with three matrices, loss the
 *             negative inner product of f(k) and v, per-token learning rate,
 *             chunk gradient summed over the chunk;
 *           - section 3.3: plain gradient-descent update, then L2 normalisation
 *             of the fast weights;
 *           - section 4: causal order (apply the state carried from previous
 *             chunks to the current chunk, then update with it) and the
 *             update-all-then-apply order for view synthesis.
 *
 * Readings where the pages leave a step open (each one is also listed with
 * the project's design notes):
 *  R1 y_t sees token t's own update (inclusive), per y_t = f(q_t, W_t) and the
 *     mini-batch sum that runs to i = t.
 *  R2 eta is per (batch, head, token) and scales that token's gradient.
 *  R3 the MSE loss carries the factor 1/2.
 *  R4 the gradient of every token of chunk c is taken at the state before the
 *     chunk's first token.
 *  R5 chunk c covers tokens [c*b, min((c+1)*b, T)); the last chunk may be short.
 *  R6 non-causal TTT-Linear: chunked updates over all K/V, then y_j = q_j W_final.
 *  R7 LaCT has no intra-chunk term: a chunk's outputs use the chunk-start
 *     weights (causal) or the final weights (non-causal).
 *  R8 LaCT L2 normalisation: each row of W1, W3 (in R^d) and of W2 (in R^hid)
 *     is rescaled to its pre-update L2 norm; a row whose new norm is exactly 0
 *     is left as is.  Off when rownorm == 0.
 *  R9 LaCT MSE variant (not used by the workloads): L = 1/2 ||f(k) - v||^2.
 *  R10 silu(z) = z * sigmoid(z); silu'(z) = s (1 + z (1 - s)), s = sigmoid(z).
 *  R11 LaCT update rules (section 3.3 names gradient descent, momentum and
 *     Muon, which maps the matrix gradient through a Newton-Schulz iteration,
 *     and gives no coefficients): momentum M <- beta M + G with step M; Muon
 *     steps lr * NS_k(M) with the textbook cubic Newton-Schulz iteration for
 *     the orthogonal polar factor started from M / ||M||_F; beta, k and lr
 *     are parameters; the row rescale of R8 follows every rule.
 *
 * Parity: every function here is pinned by tests against closed forms and
 * brute force (causal linear attention, the delta rule, one-chunk dense
 * algebra, finite-difference gradients, invariants).  Multi-chunk LaCT values
 * have no closed form on the pages: they are pinned only through their pieces.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2

/* ------------------------------------------------------------------------ */
/* TTT-Linear: f(x, W) = x W, W is d x d, row-vector convention.             */
/* ------------------------------------------------------------------------ */

/* One (batch, head) pair.  q: [Tq][d], k, v: [Tkv][d], eta: [Tkv],
 * w: [d][d] (in, out) holds the initial state on entry and the final state on
 * exit.  out: [Tq][d].  scratch: 2*d doubles + d*d doubles. */
static void ttt_linear_head(const double *q, const double *k, const double *v, const double *eta,
                            double *w, double *out, int Tq, int Tkv, int d, int chunk, int loss,
                            int order, double *scratch)
{
    double *wc = scratch;            /* chunk-start state W_c, d x d       */
    double *r = scratch + (size_t)d * d; /* per-token gradient factor, d     */
    const int causal = (order == 0);

    for (int c0 = 0; c0 < Tkv; c0 += chunk) {
        const int c1 = (c0 + chunk < Tkv) ? c0 + chunk : Tkv;
        /* R4: every gradient in this chunk is evaluated at W_c. */
        memcpy(wc, w, sizeof(double) * (size_t)d * d);
        for (int t = c0; t < c1; ++t) {
            const double *kt = k + (size_t)t * d;
            const double *vt = v + (size_t)t * d;
            /* grad_W L_t = k_t^T r_t with
             *   MSE: L = 1/2 ||k W_c - v||^2  ->  r = k_t W_c - v_t
             *   DOT: L = -(k W_c) . v         ->  r = -v_t                  */
            for (int j = 0; j < d; ++j) {
                if (loss == 1) {
                    double s = 0.0;
                    for (int i = 0; i < d; ++i) s += kt[i] * wc[(size_t)i * d + j];
                    r[j] = s - vt[j];
                } else {
                    r[j] = -vt[j];
                }
            }
            /* W <- W - eta_t * k_t^T r_t  (the running mini-batch sum of R2/R4). */
            const double et = eta[t];
            for (int i = 0; i < d; ++i) {
                const double a = et * kt[i];
                double *wi = w + (size_t)i * d;
                for (int j = 0; j < d; ++j) wi[j] -= a * r[j];
            }
            /* R1: y_t = q_t W_t, after token t's own update. */
            if (causal && t < Tq) {
                const double *qt = q + (size_t)t * d;
                double *yt = out + (size_t)t * d;
                for (int j = 0; j < d; ++j) {
                    double s = 0.0;
                    for (int i = 0; i < d; ++i) s += qt[i] * w[(size_t)i * d + j];
                    yt[j] = s;
                }
            }
        }
    }
    if (!causal) {
        /* R6: every query reads the final state. */
        for (int t = 0; t < Tq; ++t) {
            const double *qt = q + (size_t)t * d;
            double *yt = out + (size_t)t * d;
            for (int j = 0; j < d; ++j) {
                double s = 0.0;
                for (int i = 0; i < d; ++i) s += qt[i] * w[(size_t)i * d + j];
                yt[j] = s;
            }
        }
    }
}

/* q [B,H,Tq,d]; k, v [B,H,Tkv,d]; eta [B,H,Tkv]; w_init [B,H,d,d];
 * out [B,H,Tq,d]; w_final [B,H,d,d].  loss: 0 = inner product, 1 = MSE.
 * order: 0 = causal (Tq must equal Tkv), 1 = non-causal.  nthreads <= 0: default. */
int oracle_ttt_linear(const double *q, const double *k, const double *v, const double *eta,
                      const double *w_init, double *out, double *w_final, int B, int H, int Tq,
                      int Tkv, int d, int chunk, int loss, int order, int nthreads)
{
    if (B < 1 || H < 1 || Tq < 0 || Tkv < 0 || d < 1 || chunk < 1) return ORACLE_EINVAL;
    if (loss != 0 && loss != 1) return ORACLE_EINVAL;
    if (order != 0 && order != 1) return ORACLE_EINVAL;
    if (order == 0 && Tq != Tkv) return ORACLE_EINVAL;
    const int NH = B * H;
    int err = ORACLE_OK;
#ifdef _OPENMP
    /* a thread count for this loop only (the process-wide default is left as is) */
    const int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nth)
#endif
    for (int h = 0; h < NH; ++h) {
        double *scratch = (double *)malloc(sizeof(double) * ((size_t)d * d + 2 * (size_t)d));
        if (!scratch) {
            err = ORACLE_ENOMEM;
            continue;
        }
        double *w = w_final + (size_t)h * d * d;
        memcpy(w, w_init + (size_t)h * d * d, sizeof(double) * (size_t)d * d);
        ttt_linear_head(q + (size_t)h * Tq * d, k + (size_t)h * Tkv * d, v + (size_t)h * Tkv * d,
                        eta + (size_t)h * Tkv, w, out + (size_t)h * Tq * d, Tq, Tkv, d, chunk, loss,
                        order, scratch);
        free(scratch);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* LaCT SwiGLU: f(x) = W2 (silu(W1 x) * (W3 x)), column convention,          */
/* W1, W3: [hid][d] (out, in); W2: [d][hid].                                  */
/* ------------------------------------------------------------------------ */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* y = f(x) with the given weights; h1, h3: hid scratch. */
static void swiglu_apply(const double *w1, const double *w2, const double *w3, const double *x,
                         double *y, double *h1, double *h3, int d, int hid)
{
    for (int r = 0; r < hid; ++r) {
        double s1 = 0.0, s3 = 0.0;
        for (int i = 0; i < d; ++i) {
            s1 += w1[(size_t)r * d + i] * x[i];
            s3 += w3[(size_t)r * d + i] * x[i];
        }
        h1[r] = s1;
        h3[r] = s3;
    }
    for (int o = 0; o < d; ++o) {
        double s = 0.0;
        for (int r = 0; r < hid; ++r) s += w2[(size_t)o * hid + r] * (h1[r] * sigmoid(h1[r]) * h3[r]);
        y[o] = s;
    }
}

/* R8: row r of X (ncols wide) back to its pre-update norm. */
static void rownorm_restore(double *x, const double *norm_before, int nrows, int ncols)
{
    for (int r = 0; r < nrows; ++r) {
        double *row = x + (size_t)r * ncols;
        double s = 0.0;
        for (int c = 0; c < ncols; ++c) s += row[c] * row[c];
        const double n = sqrt(s);
        if (n == 0.0) continue;
        const double f = norm_before[r] / n;
        for (int c = 0; c < ncols; ++c) row[c] *= f;
    }
}

static void row_norms(const double *x, double *norm, int nrows, int ncols)
{
    for (int r = 0; r < nrows; ++r) {
        double s = 0.0;
        for (int c = 0; c < ncols; ++c) s += x[(size_t)r * ncols + c] * x[(size_t)r * ncols + c];
        norm[r] = sqrt(s);
    }
}

typedef struct {
    double *g1, *g2, *g3;       /* summed chunk gradients */
    double *h1, *h3, *a, *g, *dy, *dg, *y;
    double *n1, *n2, *n3;       /* pre-update row norms */
} lact_scratch;

/* Accumulate, at the given weights, the gradient of sum_t eta_t L_t over
 * tokens [t0, t1) into s->g1, g2, g3 (which the caller zeroed).  Explicit
 * per-token chain rule of f(x) = W2 (a * h3), a = silu(h1), h1 = W1 x, h3 = W3 x:
 *   dL/dy  = -v (inner product)  or  f(x) - v (MSE, R9), times eta_t;
 *   dW2   += dy g^T;  dg = W2^T dy;
 *   dW3   += (dg * a) x^T;  dW1 += (dg * h3 * silu'(h1)) x^T.               */
static void lact_chunk_grad(const double *w1, const double *w2, const double *w3, const double *k,
                            const double *v, const double *eta, int t0, int t1, int d, int hid,
                            int loss, lact_scratch *s)
{
    for (int t = t0; t < t1; ++t) {
        const double *x = k + (size_t)t * d;
        const double *vt = v + (size_t)t * d;
        const double et = eta[t];
        for (int r = 0; r < hid; ++r) {
            double s1 = 0.0, s3 = 0.0;
            for (int i = 0; i < d; ++i) {
                s1 += w1[(size_t)r * d + i] * x[i];
                s3 += w3[(size_t)r * d + i] * x[i];
            }
            s->h1[r] = s1;
            s->h3[r] = s3;
            s->a[r] = s1 * sigmoid(s1);
            s->g[r] = s->a[r] * s3;
        }
        if (loss == 1) {
            for (int o = 0; o < d; ++o) {
                double acc = 0.0;
                for (int r = 0; r < hid; ++r) acc += w2[(size_t)o * hid + r] * s->g[r];
                s->dy[o] = et * (acc - vt[o]);
            }
        } else {
            for (int o = 0; o < d; ++o) s->dy[o] = -et * vt[o];
        }
        for (int o = 0; o < d; ++o)
            for (int r = 0; r < hid; ++r) s->g2[(size_t)o * hid + r] += s->dy[o] * s->g[r];
        for (int r = 0; r < hid; ++r) {
            double acc = 0.0;
            for (int o = 0; o < d; ++o) acc += w2[(size_t)o * hid + r] * s->dy[o];
            s->dg[r] = acc;
        }
        for (int r = 0; r < hid; ++r) {
            const double sg = sigmoid(s->h1[r]);
            const double dsilu = sg * (1.0 + s->h1[r] * (1.0 - sg));
            const double d3 = s->dg[r] * s->a[r];
            const double d1 = s->dg[r] * s->h3[r] * dsilu;
            for (int i = 0; i < d; ++i) {
                s->g3[(size_t)r * d + i] += d3 * x[i];
                s->g1[(size_t)r * d + i] += d1 * x[i];
            }
        }
    }
}

/* Update rules (R11).  rule 0: plain gradient descent.  rule 1:
 * momentum, M <- beta M + G, step M.  rule 2: Muon, M as for momentum (M = G
 * when beta == 0), step lr * NS_k(M), where NS_k is k steps of the cubic
 * Newton-Schulz iteration for the orthogonal polar factor,
 *     X_0 = M / ||M||_F,   X_{j+1} = 1.5 X_j - 0.5 X_j (X_j^T X_j),
 * and the zero matrix maps to zero. */
typedef struct {
    int rule;
    double beta;
    int ns_steps;
    double lr;
    double *m1, *m2, *m3;   /* momentum buffers of this head (rules 1, 2 with beta != 0) */
    double *x, *gram, *prod;   /* Newton-Schulz scratch */
} lact_rule;

static void newton_schulz(double *dst, int rows, int cols, int steps, lact_rule *u)
{
    const size_t n = (size_t)rows * cols;
    double ss = 0.0;
    for (size_t i = 0; i < n; ++i) ss += dst[i] * dst[i];
    if (ss == 0.0) return;
    const double inv = 1.0 / sqrt(ss);
    for (size_t i = 0; i < n; ++i) u->x[i] = dst[i] * inv;
    for (int it = 0; it < steps; ++it) {
        /* gram = X^T X  (cols x cols) */
        for (int i = 0; i < cols; ++i)
            for (int j = 0; j < cols; ++j) {
                double acc = 0.0;
                for (int r = 0; r < rows; ++r) acc += u->x[(size_t)r * cols + i] * u->x[(size_t)r * cols + j];
                u->gram[(size_t)i * cols + j] = acc;
            }
        /* prod = X gram */
        for (int r = 0; r < rows; ++r)
            for (int j = 0; j < cols; ++j) {
                double acc = 0.0;
                for (int i = 0; i < cols; ++i) acc += u->x[(size_t)r * cols + i] * u->gram[(size_t)i * cols + j];
                u->prod[(size_t)r * cols + j] = acc;
            }
        for (size_t i = 0; i < n; ++i) u->x[i] = 1.5 * u->x[i] - 0.5 * u->prod[i];
    }
    for (size_t i = 0; i < n; ++i) dst[i] = u->x[i];
}

/* The step direction of one matrix (in place over its gradient g). */
static void rule_direction(double *g, double *m, int rows, int cols, lact_rule *u)
{
    const size_t n = (size_t)rows * cols;
    if (u->rule == 0) return;
    if (m) {
        for (size_t i = 0; i < n; ++i) {
            m[i] = u->beta * m[i] + g[i];
            g[i] = m[i];
        }
    }
    if (u->rule == 2) {
        newton_schulz(g, rows, cols, u->ns_steps, u);
        for (size_t i = 0; i < n; ++i) g[i] *= u->lr;
    }
}

/* Step W <- W - direction on the three matrices, then R8. */
static void lact_update(double *w1, double *w2, double *w3, int d, int hid, int rownorm,
                        lact_scratch *s, lact_rule *u)
{
    const size_t n13 = (size_t)hid * d, n2 = (size_t)d * hid;
    if (rownorm) {
        row_norms(w1, s->n1, hid, d);
        row_norms(w2, s->n2, d, hid);
        row_norms(w3, s->n3, hid, d);
    }
    rule_direction(s->g1, u->m1, hid, d, u);
    rule_direction(s->g2, u->m2, d, hid, u);
    rule_direction(s->g3, u->m3, hid, d, u);
    for (size_t i = 0; i < n13; ++i) w1[i] -= s->g1[i];
    for (size_t i = 0; i < n2; ++i) w2[i] -= s->g2[i];
    for (size_t i = 0; i < n13; ++i) w3[i] -= s->g3[i];
    if (rownorm) {
        rownorm_restore(w1, s->n1, hid, d);
        rownorm_restore(w2, s->n2, d, hid);
        rownorm_restore(w3, s->n3, hid, d);
    }
}

static void lact_head(const double *q, const double *k, const double *v, const double *eta,
                      double *w1, double *w2, double *w3, double *out, int Tq, int Tkv, int d,
                      int hid, int chunk, int loss, int order, int rownorm, lact_scratch *s,
                      lact_rule *u)
{
    const size_t n13 = (size_t)hid * d, n2 = (size_t)d * hid;
    const int causal = (order == 0);
    for (int c0 = 0; c0 < Tkv; c0 += chunk) {
        const int c1 = (c0 + chunk < Tkv) ? c0 + chunk : Tkv;
        if (causal) {
            /* Apply first: the chunk's queries read the state carried in (R7). */
            for (int t = c0; t < c1 && t < Tq; ++t)
                swiglu_apply(w1, w2, w3, q + (size_t)t * d, out + (size_t)t * d, s->h1, s->h3, d, hid);
        }
        memset(s->g1, 0, sizeof(double) * n13);
        memset(s->g2, 0, sizeof(double) * n2);
        memset(s->g3, 0, sizeof(double) * n13);
        lact_chunk_grad(w1, w2, w3, k, v, eta, c0, c1, d, hid, loss, s);
        lact_update(w1, w2, w3, d, hid, rownorm, s, u);
    }
    if (!causal) {
        for (int t = 0; t < Tq; ++t)
            swiglu_apply(w1, w2, w3, q + (size_t)t * d, out + (size_t)t * d, s->h1, s->h3, d, hid);
    }
}

/* q [B,H,Tq,d]; k, v [B,H,Tkv,d]; eta [B,H,Tkv];
 * w1_init, w3_init [B,H,hid,d]; w2_init [B,H,d,hid]; out [B,H,Tq,d];
 * w*_final like the inits.  loss: 0 inner product, 1 MSE.  order: 0 causal
 * (Tq == Tkv), 1 non-causal.  rownorm: 1 = R8 on, 0 = off.
 * rule: 0 gradient descent, 1 momentum, 2 Muon (see lact_rule); m1, m2, m3
 * (like w1, w2, w3) are the momentum buffers, read and updated in place, used
 * by rule 1 and by rule 2 when beta != 0 (may be NULL otherwise). */
int oracle_lact_swiglu_rule(const double *q, const double *k, const double *v, const double *eta,
                            const double *w1_init, const double *w2_init, const double *w3_init,
                            double *out, double *w1_final, double *w2_final, double *w3_final,
                            int B, int H, int Tq, int Tkv, int d, int hid, int chunk, int loss,
                            int order, int rownorm, int rule, double beta, int ns_steps, double lr,
                            double *m1, double *m2, double *m3, int nthreads)
{
    if (B < 1 || H < 1 || Tq < 0 || Tkv < 0 || d < 1 || hid < 1 || chunk < 1) return ORACLE_EINVAL;
    if (loss != 0 && loss != 1) return ORACLE_EINVAL;
    if (order != 0 && order != 1) return ORACLE_EINVAL;
    if (order == 0 && Tq != Tkv) return ORACLE_EINVAL;
    if (rule < 0 || rule > 2 || (rule == 2 && ns_steps < 0)) return ORACLE_EINVAL;
    const int use_m = rule == 1 || (rule == 2 && beta != 0.0);
    if (use_m && (!m1 || !m2 || !m3)) return ORACLE_EINVAL;
    const int NH = B * H;
    const size_t n13 = (size_t)hid * d, n2 = (size_t)d * hid;
    int err = ORACLE_OK;
#ifdef _OPENMP
    /* a thread count for this loop only (the process-wide default is left as is) */
    const int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nth)
#endif
    for (int h = 0; h < NH; ++h) {
        const size_t big = (size_t)(hid > d ? hid : d);
        const size_t nns = (rule == 2) ? 2 * n13 + big * big : 0;
        const size_t nscr = 2 * n13 + n2 + 6 * (size_t)hid + 3 * (size_t)d + 2 * (size_t)hid + (size_t)d + nns;
        double *buf = (double *)malloc(sizeof(double) * nscr);
        if (!buf) {
            err = ORACLE_ENOMEM;
            continue;
        }
        lact_scratch s;
        double *p = buf;
        s.g1 = p; p += n13;
        s.g3 = p; p += n13;
        s.g2 = p; p += n2;
        s.h1 = p; p += hid;
        s.h3 = p; p += hid;
        s.a = p; p += hid;
        s.g = p; p += hid;
        s.dg = p; p += hid;
        s.n1 = p; p += hid;
        s.n3 = p; p += hid;
        s.n2 = p; p += d;
        s.dy = p; p += d;
        s.y = p; p += d;
        lact_rule u;
        u.rule = rule;
        u.beta = beta;
        u.ns_steps = ns_steps;
        u.lr = lr;
        u.m1 = use_m ? m1 + (size_t)h * n13 : NULL;
        u.m2 = use_m ? m2 + (size_t)h * n2 : NULL;
        u.m3 = use_m ? m3 + (size_t)h * n13 : NULL;
        u.x = p; p += (rule == 2) ? n13 : 0;
        u.prod = p; p += (rule == 2) ? n13 : 0;
        u.gram = p;
        double *w1 = w1_final + (size_t)h * n13, *w3 = w3_final + (size_t)h * n13;
        double *w2 = w2_final + (size_t)h * n2;
        memcpy(w1, w1_init + (size_t)h * n13, sizeof(double) * n13);
        memcpy(w2, w2_init + (size_t)h * n2, sizeof(double) * n2);
        memcpy(w3, w3_init + (size_t)h * n13, sizeof(double) * n13);
        lact_head(q + (size_t)h * Tq * d, k + (size_t)h * Tkv * d, v + (size_t)h * Tkv * d,
                  eta + (size_t)h * Tkv, w1, w2, w3, out + (size_t)h * Tq * d, Tq, Tkv, d, hid,
                  chunk, loss, order, rownorm, &s, &u);
        free(buf);
    }
    return err;
}

int oracle_lact_swiglu(const double *q, const double *k, const double *v, const double *eta,
                       const double *w1_init, const double *w2_init, const double *w3_init,
                       double *out, double *w1_final, double *w2_final, double *w3_final, int B,
                       int H, int Tq, int Tkv, int d, int hid, int chunk, int loss, int order,
                       int rownorm, int nthreads)
{
    return oracle_lact_swiglu_rule(q, k, v, eta, w1_init, w2_init, w3_init, out, w1_final,
                                   w2_final, w3_final, B, H, Tq, Tkv, d, hid, chunk, loss, order,
                                   rownorm, 0, 0.0, 0, 0.0, NULL, NULL, NULL, nthreads);
}

/* Number of threads an OpenMP region would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
