/*
 * Q-Delta fp64 CPU oracle.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the benchmark's CPU-baseline leg load this library; the product
 * path never does.  It shares no code, header or helper with the HIP library.
 *
 * What it computes: the gated Q-Delta recurrence token by token, from the boxed
 * update on the Q-Delta reading notes page ("Q-Delta: Beyond Key-Value
 * Associative State Evolution" reading notes, section 2.4, boxed equation):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t x_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,         with x_t = k_t + lambda_t q_t  (section 2.1 table).
 *
 * State convention (same page, section 2.1 table): S is d_v x d_k, so S k is the
 * value predicted for key k.  In memory a state is row-major [d_v][d_k] (row =
 * value index, column = key index).
 *
 * The transition multiplies S from the right, so row i of the state, s (length
 * d_k), is mapped on its own:
 *
 *     s  ->  alpha s - alpha beta (s . x) k + beta v_i k
 *
 * (the matrix equation restricted to one row; only v_t[i] enters).  The code
 * evaluates exactly this expression per row, in fp64, with plain left-to-right
 * dot products, then reads out o_t[i] = s . q from the updated row.  The loops run
 * the row loop outside the time loop and hand independent rows to OpenMP threads.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (see build_oracle.py).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static double dot(const double *a, const double *b, int n)
{
    double acc = 0.0;
    int j;
    for (j = 0; j < n; ++j) acc += a[j] * b[j];
    return acc;
}

/* Row form of the boxed update for one state row s (length dk), in place:
 *     s <- alpha (s - beta (s . read) write) + beta v_i write
 * i.e. s (alpha (I - beta read write^T)) + beta v_i write^T.  Q-Delta has
 * read = x_t and write = k_t. */
static void gated_row_update(double *s, const double *read, const double *write,
                             double v_i, double alpha, double beta, int dk)
{
    const double s_read = dot(s, read, dk);                     /* (S_{t-1} x_t)_i */
    int j;
    for (j = 0; j < dk; ++j)
        s[j] = alpha * (s[j] - beta * s_read * write[j]) + beta * v_i * write[j];
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
        double *s = S + (size_t)i * dk;
        gated_row_update(s, read, write, v[i], alpha, beta, dk);
        if (o) o[i] = dot(s, q, dk);                           /* read-out from S_t */
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
            for (j = 0; j < dk; ++j) x[j] = kt[j] + la * qt[j];   /* x_t = k_t + lambda_t q_t */
            gated_row_update(s, x, kt, v[tok * dv + i], a, be, dk);
            if (o) o[tok * dv + i] = dot(s, qt, dk);          /* o_t = S_t q_t */
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
        double *s = S + (nh * dv + i) * dk;
        double x[1024];
        int j;
        for (j = 0; j < dk; ++j) x[j] = kt[j] + la * qt[j];
        gated_row_update(s, x, kt, v[nh * dv + i], a, beta[nh], dk);
        if (o) o[nh * dv + i] = dot(s, qt, dk);
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

/* The boxed update for one whole (dv x dk) state, row by row. */
static void step_state(double *S, const double *x, const double *kt, const double *vt,
                       double a, double be, int dk, int dv)
{
    int i;
    for (i = 0; i < dv; ++i)
        gated_row_update(S + (size_t)i * dk, x, kt, vt[i], a, be, dk);
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
 * Erase-then-Delta (page "Erase-then-Delta Attention" explainer, core method), in
 * this file's d_v x d_k convention (the page's K x V memory transposed).  Per token,
 * with a unit erase direction e, the page's erase (remove the state's component along
 * e) followed by its delta write along k with no beta composes to one map:
 *
 *     S_t = S_{t-1} (I - e e^T)(I - k k^T) + v k^T,      o_t = S_t q.
 *
 * Row form, expanding the product of the two projectors:
 *     s -> s - (s . e) e + (v_i - s . k + (s . e)(e . k)) k.
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
            const double se = dot(s, et, dk), sk = dot(s, kt, dk), ek = dot(et, kt, dk);
            const double coef_k = v[tok * dv + i] - sk + se * ek;
            for (j = 0; j < dk; ++j) s[j] = s[j] - se * et[j] + coef_k * kt[j];
            if (o) o[tok * dv + i] = dot(s, qt, dk);
        }
    }
    return 0;
}
