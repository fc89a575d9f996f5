/*
 * Q-Delta fp64 CPU oracle.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the benchmark's CPU-baseline leg load this library; the product
 * path never does.  It shares no code, header or helper with the HIP library.
 *
 * What it computes: the token-by-token gated Q-Delta recurrence, exactly as the
 * Q-Delta reading notes state it (page "Q-Delta: Beyond Key-Value Associative
 * State Evolution" reading notes, section 2.4 "Q-Delta 的逐步计算", the boxed
 * gated update and its teaching pseudo-code):
 *
 *     x_t       = k_t + lambda_t q_t            (mixed read direction, §2.1 table)
 *     S_prior   = alpha_t S_{t-1}               (decay first)
 *     err_t     = v_t - S_prior x_t             (error read along x_t)
 *     S_t       = S_prior + beta_t err_t k_t^T  (rank-one write along k_t)
 *     o_t       = S_t q_t                       (read-out uses the updated state)
 *
 * State convention (same page, §2.1 table): S is d_v x d_k, so the prediction
 * along a key is S k and the read-out is S q.  In memory a state is row-major
 * [d_v][d_k] (row = value index, column = key index).
 *
 * The transition acts on S from the right (S_prior (I - beta x k^T)), so each row
 * of S evolves on its own: row i only sees v_t[i].  The loops below therefore run
 * the row loop outside the time loop and hand independent rows to OpenMP
 * threads.  Within a row the arithmetic is the pseudo-code above, step for step,
 * in fp64, with no reassociation beyond plain left-to-right dot products.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (see build_oracle.py).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* Advance one row s (length dk) by one token.
 *   read  : direction the error is read along (x_t for Q-Delta)
 *   write : direction the correction is written along (k_t for Q-Delta)
 * Returns the post-update read-out s . q (the row's entry of o_t = S_t q_t). */
static double advance_row(double *s, const double *read, const double *write,
                          const double *q, double v_i, double alpha, double beta,
                          int dk)
{
    int j;
    double pred = 0.0, err, out = 0.0;
    for (j = 0; j < dk; ++j) s[j] = alpha * s[j];          /* S_prior = alpha S   */
    for (j = 0; j < dk; ++j) pred += s[j] * read[j];       /* (S_prior x)_i       */
    err = v_i - pred;                                      /* error_i             */
    for (j = 0; j < dk; ++j) s[j] = s[j] + beta * err * write[j]; /* + beta err k^T */
    for (j = 0; j < dk; ++j) out += s[j] * q[j];           /* o_i = (S_t q)_i     */
    return out;
}

/* One step with an explicit read direction and write direction, for a single
 * state S [dv][dk] (updated in place) and one token.  o (length dv) may be NULL.
 * Q-Delta is the case read = k + lambda q, write = k.  The general form lets a
 * test drive the step the QED reading notes' two-dimensional example describes
 * (page "The Query Knows What to Forget" reading notes, §2.4), where the read
 * direction differs from the write direction. */
void oracle_step_rw(double *S, const double *read, const double *write,
                    const double *v, const double *q, double alpha, double beta,
                    double *o, int dk, int dv)
{
    int i;
    for (i = 0; i < dv; ++i) {
        double out = advance_row(S + (size_t)i * dk, read, write, q, v[i], alpha, beta, dk);
        if (o) o[i] = out;
    }
}

/* Full layer forward by the recurrence.
 *   q, k   : [B][T][H][dk]          v, o : [B][T][H][dv]
 *   alpha, beta, lam : [B][T][H]    (alpha NULL means alpha == 1, lam NULL means lambda == 0)
 *   S0     : [B][H][dv][dk] or NULL (zero initial state)
 *   S_T    : [B][H][dv][dk] output, required; also used as the working state
 *   o      : may be NULL (state only)
 *   nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument. */
int oracle_qdelta_fwd(const double *q, const double *k, const double *v,
                      const double *alpha, const double *beta, const double *lam,
                      const double *S0, double *o, double *S_T,
                      int B, int T, int H, int dk, int dv, int nthreads)
{
    long long unit, n_units;
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1 || dk > 1024) return -1;
    if (!S_T) return -1;
    if ((long long)B * T * H > 0 && (!q || !k || !v || !beta)) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    n_units = (long long)B * H * dv;           /* one unit = one row of one (b,h) state */
#pragma omp parallel for schedule(dynamic, 8) num_threads(nthreads)
    for (unit = 0; unit < n_units; ++unit) {
        int b = (int)(unit / ((long long)H * dv));
        int h = (int)((unit / dv) % H);
        int i = (int)(unit % dv);
        double *s = S_T + (((size_t)b * H + h) * dv + i) * dk;
        double x[1024];
        int t, j;
        if (S0) memcpy(s, S0 + (((size_t)b * H + h) * dv + i) * dk, sizeof(double) * dk);
        else memset(s, 0, sizeof(double) * dk);
        for (t = 0; t < T; ++t) {
            size_t tok = ((size_t)b * T + t) * H + h;      /* token-head index */
            const double *qt = q + tok * dk;
            const double *kt = k + tok * dk;
            double a = alpha ? alpha[tok] : 1.0;
            double be = beta[tok];
            double la = lam ? lam[tok] : 0.0;
            double out;
            for (j = 0; j < dk; ++j) x[j] = kt[j] + la * qt[j];   /* x_t = k_t + lambda_t q_t */
            out = advance_row(s, x, kt, qt, v[tok * dv + i], a, be, dk);
            if (o) o[tok * dv + i] = out;
        }
    }
    return 0;
}

/* One recurrent decode step for N independent sequences x H heads.
 *   q, k : [N][H][dk]   v, o : [N][H][dv]   alpha, beta, lam : [N][H]
 *   S    : [N][H][dv][dk], updated in place.   o may be NULL.
 * Returns 0, or -1 on a bad argument. */
int oracle_qdelta_step(const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta, const double *lam,
                       double *S, double *o, int N, int H, int dk, int dv, int nthreads)
{
    long long unit, n_units;
    if (N < 0 || H < 0 || dk < 1 || dv < 1 || dk > 1024) return -1;
    if ((long long)N * H > 0 && (!q || !k || !v || !beta || !S)) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    n_units = (long long)N * H * dv;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (unit = 0; unit < n_units; ++unit) {
        size_t nh = (size_t)(unit / dv);
        int i = (int)(unit % dv);
        const double *qt = q + nh * dk;
        const double *kt = k + nh * dk;
        double a = alpha ? alpha[nh] : 1.0;
        double la = lam ? lam[nh] : 0.0;
        double x[1024], out;
        int j;
        for (j = 0; j < dk; ++j) x[j] = kt[j] + la * qt[j];
        out = advance_row(S + (nh * dv + i) * dk, x, kt, qt, v[nh * dv + i], a, beta[nh], dk);
        if (o) o[nh * dv + i] = out;
    }
    return 0;
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------ backward
 * Gradients of the layer forward above, by reverse-mode differentiation of the
 * recurrence one token at a time.  The pages state the forward only; this is the
 * adjoint of each of its lines, derived by hand (there is nothing more to it than
 * the chain rule).  For token t, with P = S_{t-1} the entry state:
 *
 *     forward                          adjoint (G = dLoss/dS_t, accumulated)
 *     x   = k + lam q                  G    += do_t q^T            (o_t = S_t q)
 *     pre = alpha P x                  dq   += S_t^T do_t
 *     u   = v - pre                    gk    = G k
 *     S_t = alpha P + beta u k^T       dbeta = u . gk ;  du = beta gk ;  dv = du
 *     o_t = S_t q                      dk   += beta G^T u
 *                                      dalpha = <G, P> - du . (P x)
 *                                      dx    = -alpha P^T du
 *                                      dk   += dx ; dq += lam dx ; dlam = q . dx
 *                                      G     <- alpha G - alpha du x^T   (= dLoss/dS_{t-1})
 *
 * and dS0 is G after the first token.  The entry states are recomputed, not
 * inverted: the forward keeps a copy of the state every SEG tokens, and the
 * reverse sweep regenerates the SEG states of one stretch from its copy before
 * walking back through it.  That changes memory use, not the arithmetic.
 */
#define ORACLE_BWD_SEG 64

/* S <- alpha S + beta (v - alpha S x) k^T for one (dv x dk) state (the same step as
 * advance_row, written for a whole state). */
static void step_state(double *S, const double *x, const double *kt, const double *vt,
                       double a, double be, int dk, int dv)
{
    int i;
    for (i = 0; i < dv; ++i)
        advance_row(S + (size_t)i * dk, x, kt, kt, vt[i], a, be, dk);
}

/* Backward of oracle_qdelta_fwd for the loss sum(o * dO) + sum(S_T * dST).
 *   q, k, v, alpha, beta, lam, S0 : as oracle_qdelta_fwd (alpha/lam/S0 may be NULL)
 *   dO  : [B][T][H][dv]   dST : [B][H][dv][dk] or NULL (zero)
 *   outputs dq, dk [B][T][H][dk]; dv [B][T][H][dv]; dalpha, dbeta, dlam [B][T][H];
 *   dS0 [B][H][dv][dk].  All required (dalpha and dlam are the gradients at the
 *   values used, alpha = 1 and lambda = 0 when those inputs are NULL).
 * One OpenMP unit per (b, h).  Returns 0, -1 on a bad argument, -2 if memory runs out. */
int oracle_qdelta_bwd(const double *q, const double *k, const double *v,
                      const double *alpha, const double *beta, const double *lam,
                      const double *S0, const double *dO, const double *dST,
                      double *dq, double *dk, double *dv, double *dalpha, double *dbeta,
                      double *dlam, double *dS0,
                      int B, int T, int H, int dkn, int dvn, int nthreads)
{
    long long unit, n_units;
    int failed = 0;
    if (B < 0 || T < 0 || H < 0 || dkn < 1 || dvn < 1 || dkn > 1024 || dvn > 1024) return -1;
    if (!dq || !dk || !dv || !dalpha || !dbeta || !dlam || !dS0) return -1;
    if ((long long)B * T * H > 0 && (!q || !k || !v || !beta || !dO)) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    n_units = (long long)B * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (unit = 0; unit < n_units; ++unit) {
        const int b = (int)(unit / H), h = (int)(unit % H);
        const size_t ns = (size_t)dvn * dkn;
        const int nseg = (T + ORACLE_BWD_SEG - 1) / ORACLE_BWD_SEG;
        double *ckpt = malloc(sizeof(double) * ns * (size_t)(nseg > 0 ? nseg : 1));
        double *states = malloc(sizeof(double) * ns * (ORACLE_BWD_SEG + 1));
        double *G = malloc(sizeof(double) * ns);
        double x[1024], gk[1024], u[1024], du[1024], px[1024], dx[1024];
        double *S;
        int t, i, j, sg;
        if (!ckpt || !states || !G) {
            free(ckpt); free(states); free(G);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        /* forward, keeping the state at the start of every stretch */
        S = states;
        if (S0) memcpy(S, S0 + unit * ns, sizeof(double) * ns);
        else memset(S, 0, sizeof(double) * ns);
        for (t = 0; t < T; ++t) {
            size_t tok = ((size_t)b * T + t) * H + h;
            double la = lam ? lam[tok] : 0.0;
            if (t % ORACLE_BWD_SEG == 0) memcpy(ckpt + (size_t)(t / ORACLE_BWD_SEG) * ns, S, sizeof(double) * ns);
            for (j = 0; j < dkn; ++j) x[j] = k[tok * dkn + j] + la * q[tok * dkn + j];
            step_state(S, x, k + tok * dkn, v + tok * dvn, alpha ? alpha[tok] : 1.0, beta[tok], dkn, dvn);
        }
        /* reverse sweep */
        if (dST) memcpy(G, dST + unit * ns, sizeof(double) * ns);
        else memset(G, 0, sizeof(double) * ns);
        for (sg = nseg - 1; sg >= 0; --sg) {
            const int t0 = sg * ORACLE_BWD_SEG;
            const int t1 = (t0 + ORACLE_BWD_SEG < T) ? t0 + ORACLE_BWD_SEG : T;
            memcpy(states, ckpt + (size_t)sg * ns, sizeof(double) * ns);
            for (t = t0; t < t1; ++t) {   /* states[t - t0] = S_{t-1} (entry state of token t) */
                size_t tok = ((size_t)b * T + t) * H + h;
                double la = lam ? lam[tok] : 0.0;
                double *nxt = states + (size_t)(t - t0 + 1) * ns;
                memcpy(nxt, states + (size_t)(t - t0) * ns, sizeof(double) * ns);
                for (j = 0; j < dkn; ++j) x[j] = k[tok * dkn + j] + la * q[tok * dkn + j];
                step_state(nxt, x, k + tok * dkn, v + tok * dvn, alpha ? alpha[tok] : 1.0, beta[tok], dkn, dvn);
            }
            for (t = t1 - 1; t >= t0; --t) {
                size_t tok = ((size_t)b * T + t) * H + h;
                const double *qt = q + tok * dkn, *kt = k + tok * dkn, *vt = v + tok * dvn;
                const double *dot = dO + tok * dvn;
                const double *P = states + (size_t)(t - t0) * ns;       /* S_{t-1} */
                const double *St = states + (size_t)(t - t0 + 1) * ns;  /* S_t     */
                double a = alpha ? alpha[tok] : 1.0, be = beta[tok], la = lam ? lam[tok] : 0.0;
                double acc, da, db, dl;
                double *dqt = dq + tok * dkn, *dkt = dk + tok * dkn, *dvt = dv + tok * dvn;
                for (j = 0; j < dkn; ++j) x[j] = kt[j] + la * qt[j];
                /* o_t = S_t q */
                for (i = 0; i < dvn; ++i)
                    for (j = 0; j < dkn; ++j) G[(size_t)i * dkn + j] += dot[i] * qt[j];
                for (j = 0; j < dkn; ++j) {
                    acc = 0.0;
                    for (i = 0; i < dvn; ++i) acc += St[(size_t)i * dkn + j] * dot[i];
                    dqt[j] = acc;
                }
                /* S_t = alpha P + beta u k^T,  u = v - alpha P x */
                for (i = 0; i < dvn; ++i) {
                    double s1 = 0.0, s2 = 0.0;
                    for (j = 0; j < dkn; ++j) {
                        s1 += G[(size_t)i * dkn + j] * kt[j];
                        s2 += P[(size_t)i * dkn + j] * x[j];
                    }
                    gk[i] = s1;
                    px[i] = s2;
                    u[i] = vt[i] - a * s2;
                }
                db = 0.0;
                for (i = 0; i < dvn; ++i) db += u[i] * gk[i];
                for (i = 0; i < dvn; ++i) {
                    du[i] = be * gk[i];
                    dvt[i] = du[i];
                }
                for (j = 0; j < dkn; ++j) {
                    acc = 0.0;
                    for (i = 0; i < dvn; ++i) acc += G[(size_t)i * dkn + j] * u[i];
                    dkt[j] = be * acc;
                }
                da = 0.0;
                for (i = 0; i < dvn; ++i)
                    for (j = 0; j < dkn; ++j) da += G[(size_t)i * dkn + j] * P[(size_t)i * dkn + j];
                for (i = 0; i < dvn; ++i) da -= du[i] * px[i];
                for (j = 0; j < dkn; ++j) {
                    acc = 0.0;
                    for (i = 0; i < dvn; ++i) acc += P[(size_t)i * dkn + j] * du[i];
                    dx[j] = -a * acc;
                }
                dl = 0.0;
                for (j = 0; j < dkn; ++j) {
                    dkt[j] += dx[j];
                    dqt[j] += la * dx[j];
                    dl += qt[j] * dx[j];
                }
                dalpha[tok] = da;
                dbeta[tok] = db;
                dlam[tok] = dl;
                /* dLoss/dS_{t-1} */
                for (i = 0; i < dvn; ++i)
                    for (j = 0; j < dkn; ++j)
                        G[(size_t)i * dkn + j] = a * G[(size_t)i * dkn + j] - a * du[i] * x[j];
            }
        }
        memcpy(dS0 + unit * ns, G, sizeof(double) * ns);
        free(ckpt); free(states); free(G);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------ QED / GDN-2
 * The QED reading notes' update (page "The Query Knows What to Forget" reading notes,
 * §2.1 and §2.2, the boxed update), written in this file's state convention: their
 * state is K x V, the transpose of ours, so S here is d_v x d_k and their S^T x is
 * our S x.  Per token, with per-key-channel log decay g (d_k), erase gate b (d_k),
 * write gate w (d_v) and the head's strength lambda_h:
 *
 *     S_bar = S_{t-1} Diag(exp g)              (decay each key column)
 *     u     = b . q                             (gate the query first ...)
 *     d     = u - k (k^T u)                     (... then project off k; |k| = 1)
 *     a     = b . k + lambda_h d                (erase / read direction)
 *     r     = w . v - S_bar a                   (residual, d_v)
 *     S_t   = S_bar + r k^T                     (rank-one write along k)
 *     o_t   = S_t q
 *
 * lambda_h = 0 is GDN-2 (same page, §2.1).  Rows of S evolve independently.
 */
int oracle_qed_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *b, const double *w, const double *lam_h,
                   const double *S0, double *o, double *S_T,
                   int B, int T, int H, int dk, int dv, int nthreads)
{
    long long unit, n_units;
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1 || dk > 1024) return -1;
    if (!S_T) return -1;
    if ((long long)B * T * H > 0 && (!q || !k || !v || !g || !b || !w || !lam_h)) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    n_units = (long long)B * H * dv;
#pragma omp parallel for schedule(dynamic, 8) num_threads(nthreads)
    for (unit = 0; unit < n_units; ++unit) {
        int bb = (int)(unit / ((long long)H * dv));
        int h = (int)((unit / dv) % H);
        int i = (int)(unit % dv);
        double *s = S_T + (((size_t)bb * H + h) * dv + i) * dk;
        double u[1024], a[1024];
        int t, j;
        if (S0) memcpy(s, S0 + (((size_t)bb * H + h) * dv + i) * dk, sizeof(double) * dk);
        else memset(s, 0, sizeof(double) * dk);
        for (t = 0; t < T; ++t) {
            size_t tok = ((size_t)bb * T + t) * H + h;
            const double *qt = q + tok * dk, *kt = k + tok * dk;
            const double *gt = g + tok * dk, *bt = b + tok * dk;
            double ku = 0.0, pred = 0.0, r, out = 0.0;
            for (j = 0; j < dk; ++j) u[j] = bt[j] * qt[j];
            for (j = 0; j < dk; ++j) ku += kt[j] * u[j];
            for (j = 0; j < dk; ++j) a[j] = bt[j] * kt[j] + lam_h[h] * (u[j] - kt[j] * ku);
            for (j = 0; j < dk; ++j) s[j] = s[j] * exp(gt[j]);              /* S_bar */
            for (j = 0; j < dk; ++j) pred += s[j] * a[j];                     /* (S_bar a)_i */
            r = w[tok * dv + i] * v[tok * dv + i] - pred;
            for (j = 0; j < dk; ++j) s[j] = s[j] + r * kt[j];                 /* + r k^T */
            for (j = 0; j < dk; ++j) out += s[j] * qt[j];
            if (o) o[tok * dv + i] = out;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ EDA
 * Erase-then-Delta (page "Erase-then-Delta Attention" explainer, core method, the
 * two-step pseudo-code), in this file's d_v x d_k convention (the page's K x V memory
 * transposed).  Per token, with a unit erase direction e:
 *
 *     S <- S - (S e) e^T                   (step 1: zero the component along e)
 *     S <- S + (v - S k) k^T               (step 2: delta write along k; no beta)
 *     o  = S q                             (read-out from the updated state)
 *
 * Rows of S evolve independently. */
int oracle_eda_fwd(const double *q, const double *k, const double *v, const double *e,
                   const double *S0, double *o, double *S_T,
                   int B, int T, int H, int dk, int dv, int nthreads)
{
    long long unit, n_units;
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1) return -1;
    if (!S_T) return -1;
    if ((long long)B * T * H > 0 && (!q || !k || !v || !e)) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    n_units = (long long)B * H * dv;
#pragma omp parallel for schedule(dynamic, 8) num_threads(nthreads)
    for (unit = 0; unit < n_units; ++unit) {
        int bb = (int)(unit / ((long long)H * dv));
        int h = (int)((unit / dv) % H);
        int i = (int)(unit % dv);
        double *s = S_T + (((size_t)bb * H + h) * dv + i) * dk;
        int t, j;
        if (S0) memcpy(s, S0 + (((size_t)bb * H + h) * dv + i) * dk, sizeof(double) * dk);
        else memset(s, 0, sizeof(double) * dk);
        for (t = 0; t < T; ++t) {
            size_t tok = ((size_t)bb * T + t) * H + h;
            const double *qt = q + tok * dk, *kt = k + tok * dk, *et = e + tok * dk;
            double se = 0.0, sk = 0.0, err, out = 0.0;
            for (j = 0; j < dk; ++j) se += s[j] * et[j];               /* (S e)_i */
            for (j = 0; j < dk; ++j) s[j] = s[j] - se * et[j];        /* step 1   */
            for (j = 0; j < dk; ++j) sk += s[j] * kt[j];               /* (S k)_i */
            err = v[tok * dv + i] - sk;
            for (j = 0; j < dk; ++j) s[j] = s[j] + err * kt[j];       /* step 2   */
            for (j = 0; j < dk; ++j) out += s[j] * qt[j];
            if (o) o[tok * dv + i] = out;
        }
    }
    return 0;
}
