/*
 * oracle.c -- plain float64 CPU reference of the matrix-state affine scan.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark load this library.  It
 * shares no source, header, table or helper with the GPU library.
 *
 * What it computes (one head; rows of S are value channels i, columns are key
 * channels j; S has d_v rows and d_k columns):
 *
 *   S_t = S_{t-1} E_t + f_t,     o_t = S_t q_t            (inclusive read-out)
 *
 * gated delta rule (mode 0):  E_t = alpha_t (I - beta_t k_t k_t^T),
 *                             f_t = beta_t v_t k_t^T
 * gated linear attention (mode 1):  E_t = alpha_t I,  f_t = v_t k_t^T
 * gated delta rule with separate erase and write strengths (mode 2):
 *                             E_t = alpha_t (I - be_t k_t k_t^T),
 *                             f_t = bw_t v_t k_t^T
 *   (PRISM's write-forget decoupling, gist.science explainer 2.1: the forget
 *   operator stays the Gated-DeltaNet rank-1 form while the write is free; a
 *   token with alpha = 1, be = 0 is a pure write, which is how PRISM's rank-L
 *   corrections enter the scan)
 * gated delta rule with a diagonal gate (mode 3):
 *                             E_t = diag(a_t) (I - beta_t k_t k_t^T),
 *                             f_t = beta_t v_t k_t^T
 * gated linear attention with a diagonal gate (mode 4):
 *                             E_t = diag(a_t),  f_t = v_t k_t^T
 *   (the prefix-scan notes, key design 2, list the diagonal gate among the
 *   forms E_t takes; a_t holds one decay per key channel)
 *
 * Sources:
 *  - "Sequential Parallel Duality in Prefix Scannable Models" (papernotes.org
 *    ICLR 2026 notes), key design 2: an efficient layer is an affine state
 *    update s_t = E_t |> s_{t-1} + f_t whose coefficients depend only on the
 *    current token; the second component of the running monoid product is the
 *    recurrent state, so the left-to-right fold below IS the scan's result.
 *    Key design 1: inference is one state update per token.
 *  - "PRISM: Parallel Residual Iterative Sequence Model" (gist.science
 *    explainer), Resume Technique 2.1: the state update is written
 *    S_t = S_{t-1} A_t + B_t with the forget operator A_t a structured rank-1
 *    form identical to Gated DeltaNet, and 2.2: S_{t-1} k_t is the value the
 *    state currently recalls for key k_t (so S maps keys to values and E acts
 *    on the key index).
 *  - PRISM article (banbantang.com), section 1(4): a global scalar gate decays
 *    the whole state, a rank-1 term forgets selectively along k, and each token
 *    writes one rank-1 outer product.  The page's formula itself was lost in
 *    extraction; E_t and f_t above are the reading those three statements fix.
 *    Gated linear attention is the scalar-gate member of the family listed in
 *    key design 2 of the first page (Katharopoulos et al. for the ungated case).
 *
 * Arithmetic: each token is applied exactly as written above, per row i:
 *   a_i   = sum_j S_ij k_j                       (row of S_{t-1} k_t)
 *   S_ij <- alpha (S_ij - beta a_i k_j) + beta v_i k_j      [gdn]
 *   S_ij <- alpha S_ij + v_i k_j                            [gla]
 *   S_ij <- alpha (S_ij - be a_i k_j) + bw v_i k_j          [gdn, split strengths]
 *   X_ij  = a_j S_ij;  S_ij <- X_ij - beta (X k)_i k_j + beta v_i k_j   [gdn, diagonal gate]
 *   S_ij <- a_j S_ij + v_i k_j                              [gla, diagonal gate]
 *   o_i   = sum_j S_ij q_j                       (row of S_t q_t)
 * Inputs arrive as float32 (bfloat16 inputs are exact in float32) and are
 * widened exactly to float64.  Rows of S are independent, so work is split over
 * (head, block of rows) across threads; every row sees the same sequence of
 * operations whatever the split, so results do not depend on thread count.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -pthread
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_GDN = 0, ORACLE_GLA = 1, ORACLE_GDN_EW = 2, ORACLE_GDN_DIAG = 3, ORACLE_GLA_DIAG = 4 };

typedef struct {
    int mode;
    int64_t BH, T;
    int dk, dv;
    const float *q, *k, *v, *alpha, *beta;
    const double *S0;
    double *o, *ST;
    int row_blocks;
    int64_t n_items;
    int64_t next;        /* shared work counter */
    int failed;
} job_t;

/* Apply tokens 0..T-1 of head h to rows [r0, r1) of its state. */
static int run_rows(const job_t *J, int64_t h, int r0, int r1)
{
    const int dk = J->dk, dv = J->dv;
    const int64_t T = J->T;
    const int nrows = r1 - r0;
    double *S = (double *)malloc(sizeof(double) * (size_t)nrows * (size_t)dk);
    if (!S) return -1;
    for (int r = 0; r < nrows; ++r)
        for (int j = 0; j < dk; ++j)
            S[(size_t)r * dk + j] = J->S0 ? J->S0[((size_t)h * dv + r0 + r) * dk + j] : 0.0;

    for (int64_t t = 0; t < T; ++t) {
        const size_t tok = (size_t)(h * T + t);
        const float *qt = J->q + tok * dk;
        const float *kt = J->k + tok * dk;
        const float *vt = J->v + tok * dv;
        const int diag = J->mode == ORACLE_GDN_DIAG || J->mode == ORACLE_GLA_DIAG;
        const double al = diag ? 0.0 : (double)J->alpha[tok];
        const float *ad = diag ? J->alpha + tok * dk : NULL;   /* per-key-channel decay */
        /* erase and write strengths; mode 2 reads them from two planes of BH*T */
        const double be = (J->mode != ORACLE_GLA && J->mode != ORACLE_GLA_DIAG) ? (double)J->beta[tok] : 0.0;
        const double bw = J->mode == ORACLE_GDN_EW ? (double)J->beta[(size_t)(J->BH * T) + tok] : be;
        for (int r = 0; r < nrows; ++r) {
            double *Si = S + (size_t)r * dk;
            const double vi = (double)vt[r0 + r];
            if (diag) {
                for (int j = 0; j < dk; ++j) Si[j] *= (double)ad[j];
                if (J->mode == ORACLE_GDN_DIAG) {
                    double a = 0.0;
                    for (int j = 0; j < dk; ++j) a += Si[j] * (double)kt[j];
                    for (int j = 0; j < dk; ++j) Si[j] = Si[j] - be * a * (double)kt[j] + be * vi * (double)kt[j];
                } else {
                    for (int j = 0; j < dk; ++j) Si[j] += vi * (double)kt[j];
                }
            } else if (J->mode != ORACLE_GLA) {
                double a = 0.0;
                for (int j = 0; j < dk; ++j) a += Si[j] * (double)kt[j];
                for (int j = 0; j < dk; ++j)
                    Si[j] = al * (Si[j] - be * a * (double)kt[j]) + bw * vi * (double)kt[j];
            } else {
                for (int j = 0; j < dk; ++j) Si[j] = al * Si[j] + vi * (double)kt[j];
            }
            double oi = 0.0;
            for (int j = 0; j < dk; ++j) oi += Si[j] * (double)qt[j];
            if (J->o) J->o[tok * dv + r0 + r] = oi;
        }
    }
    if (J->ST)
        memcpy(J->ST + ((size_t)h * dv + r0) * dk, S, sizeof(double) * (size_t)nrows * dk);
    free(S);
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    for (;;) {
        int64_t it = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (it >= J->n_items) break;
        const int64_t h = it / J->row_blocks;
        const int b = (int)(it % J->row_blocks);
        const int per = (J->dv + J->row_blocks - 1) / J->row_blocks;
        const int r0 = b * per;
        const int r1 = r0 + per < J->dv ? r0 + per : J->dv;
        if (r0 < r1 && run_rows(J, h, r0, r1) != 0) __atomic_store_n(&J->failed, 1, __ATOMIC_RELAXED);
    }
    return NULL;
}

/*
 * Full-sequence scan of BH independent heads.
 *   q, k: [BH, T, dk] float32     v: [BH, T, dv] float32
 *   alpha: [BH, T] float32; [BH, T, dk] float32 (modes 3, 4: one decay per key channel)
 *   beta: [BH, T] float32 (modes 0, 3); ignored, may be NULL (modes 1, 4); [2, BH, T]
 *         float32 (mode 2: erase strengths, then write strengths)
 *   S0: [BH, dv, dk] float64 or NULL (zero state)
 *   o:  [BH, T, dv] float64 or NULL (not stored; still computed)
 *   ST: [BH, dv, dk] float64 or NULL
 * Returns the number of threads used (>= 1), or -1 on bad arguments or
 * allocation failure.
 */
int oracle_scan_f64(int mode, int64_t BH, int64_t T, int dk, int dv,
                    const float *q, const float *k, const float *v,
                    const float *alpha, const float *beta, const double *S0,
                    double *o, double *ST, int nthreads)
{
    if (mode < ORACLE_GDN || mode > ORACLE_GLA_DIAG || BH < 0 || T < 0 || dk <= 0 || dv <= 0)
        return -1;
    if (mode != ORACLE_GLA && mode != ORACLE_GLA_DIAG && !beta && BH * T > 0) return -1;
    if (BH * T > 0 && (!q || !k || !v || !alpha)) return -1;
    if (nthreads < 1) nthreads = 1;

    job_t J;
    memset(&J, 0, sizeof J);
    J.mode = mode; J.BH = BH; J.T = T; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.S0 = S0;
    J.o = o; J.ST = ST;
    /* enough (head, row-block) items to keep every thread busy */
    int rb = 1;
    while (BH * rb < 2 * (int64_t)nthreads && rb < dv) rb *= 2;
    J.row_blocks = rb;
    J.n_items = BH * rb;
    if (J.n_items == 0) return 1;
    if ((int64_t)nthreads > J.n_items) nthreads = (int)J.n_items;

    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -1;
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    worker(&J);
    for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    return J.failed ? -1 : started + 1;
}

/*
 * One token for each of N independent states, state updated in place:
 *   q, k: [N, dk]   v: [N, dv]   alpha: [N] ([N, dk] in modes 3, 4)
 *   beta: [N] ([2, N] in mode 2)
 *   S: [N, dv, dk] float64
 *   o: [N, dv] float64 = S_new q
 * Same arithmetic as oracle_scan_f64 with T = 1 (the per-token update of the
 * sequential view, key design 1 of the prefix-scan notes).
 */
int oracle_decode_f64(int mode, int64_t N, int dk, int dv,
                      const float *q, const float *k, const float *v,
                      const float *alpha, const float *beta,
                      double *S, double *o, int nthreads)
{
    return oracle_scan_f64(mode, N, 1, dk, dv, q, k, v, alpha, beta, S, o, S, nthreads);
}

/*
 * Gradient of the scan (reverse mode through the token recurrence above).
 *
 * The loss is L = sum_t <dO_t, o_t> + <dST, S_T>: dO and dST are the gradients
 * arriving at the outputs.  The prefix-scan notes (key design 1) give the
 * sequential view, one state update per token; its chain rule, per row i of S
 * (a row only meets its own v_i, and meets k, q, the gates and the strengths),
 * is written here with the decay as a vector d_t over key channels (d_t = a_t
 * for modes 3, 4 and alpha_t in every channel for modes 0, 1):
 *
 *   forward   x = d_t * s_{t-1}            (elementwise)
 *             p = x . k_t
 *             s_t = x + beta_t (v_ti - p) k_t       [delta rule, modes 0, 3]
 *             s_t = x - be_t p k_t + bw_t v_ti k_t  [split strengths, mode 2]
 *             s_t = x + v_ti k_t                    [linear attention, modes 1, 4]
 *             o_ti = s_t . q_t
 *   backward  with y the gradient reaching s_t (dST's row at t = T):
 *             dq_t += dO_ti s_t,   y += dO_ti q_t
 *             delta rule:  yk = y . k_t
 *                          dv_ti = beta_t yk
 *                          dbeta_t += yk (v_ti - p)
 *                          dk_t += beta_t (v_ti - p) y - beta_t yk x
 *                          dx = y - beta_t yk k_t
 *             split strengths:  dv_ti = bw_t yk,  dbe_t -= yk p,  dbw_t += yk v_ti,
 *                               dk_t += (bw_t v_ti - be_t p) y - be_t yk x,  dx = y - be_t yk k_t
 *             linear attention:  dv_ti = y . k_t,  dk_t += v_ti y,  dx = y
 *             dd_t += dx * s_{t-1}  (summed over key channels for a scalar gate)
 *             y <- dx * d_t        (the gradient reaching s_{t-1})
 *   and dS0's row is the final y.
 * The row's states s_0 .. s_T are kept (T + 1 rows of d_k) so that the
 * backward sweep reads s_{t-1} and s_t as stored.  Rows are taken in order
 * 0 .. d_v - 1 and the shared gradients (dq, dk, dalpha, dbeta) accumulate in
 * that order, one thread per head, so results do not depend on thread count.
 * Modes 0 to 4; every input is float64 (no rounding on the way in), so
 * finite differences of the same function can check it.
 */
typedef struct {
    int mode;
    int64_t BH, T;
    int dk, dv;
    const double *q, *k, *v, *alpha, *beta, *S0, *dO, *dST;
    double *gq, *gk, *gv, *galpha, *gbeta, *gS0;
    int64_t next;
    int failed;
} bjob_t;

static int bwd_head(const bjob_t *J, int64_t h)
{
    const int dk = J->dk, dv = J->dv;
    const int64_t T = J->T;
    const int diag = J->mode == ORACLE_GDN_DIAG || J->mode == ORACLE_GLA_DIAG;
    const int delta = J->mode == ORACLE_GDN || J->mode == ORACLE_GDN_DIAG || J->mode == ORACLE_GDN_EW;
    const int split = J->mode == ORACLE_GDN_EW;
    const int da = diag ? dk : 1;  /* decay entries per token */
    const size_t wplane = (size_t)(J->BH * T);  /* offset of the write-strength plane (mode 2) */
    double *traj = (double *)malloc(sizeof(double) * (size_t)(T + 1) * (size_t)dk);
    double *x = (double *)malloc(sizeof(double) * (size_t)dk);
    double *y = (double *)malloc(sizeof(double) * (size_t)dk);
    double *dx = (double *)malloc(sizeof(double) * (size_t)dk);
    if (!traj || !x || !y || !dx) {
        free(traj); free(x); free(y); free(dx);
        return -1;
    }
    const size_t tok0 = (size_t)(h * T);
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < dk; ++j) {
            J->gq[(tok0 + t) * dk + j] = 0.0;
            J->gk[(tok0 + t) * dk + j] = 0.0;
        }
        for (int j = 0; j < da; ++j) J->galpha[(tok0 + t) * da + j] = 0.0;
        if (J->gbeta) J->gbeta[tok0 + t] = 0.0;
        if (split) J->gbeta[wplane + tok0 + t] = 0.0;
    }
    for (int i = 0; i < dv; ++i) {
        const size_t srow = ((size_t)h * dv + i) * dk;
        for (int j = 0; j < dk; ++j) traj[j] = J->S0 ? J->S0[srow + j] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const size_t tok = tok0 + (size_t)t;
            const double *kt = J->k + tok * dk;
            const double *s0 = traj + (size_t)t * dk;
            double *s1 = traj + (size_t)(t + 1) * dk;
            const double vi = J->v[tok * dv + i];
            for (int j = 0; j < dk; ++j) x[j] = (diag ? J->alpha[tok * dk + j] : J->alpha[tok]) * s0[j];
            if (delta) {
                const double be = J->beta[tok];
                const double bw = split ? J->beta[wplane + tok] : be;
                double p = 0.0;
                for (int j = 0; j < dk; ++j) p += x[j] * kt[j];
                for (int j = 0; j < dk; ++j) s1[j] = x[j] + (bw * vi - be * p) * kt[j];
            } else {
                for (int j = 0; j < dk; ++j) s1[j] = x[j] + vi * kt[j];
            }
        }
        for (int j = 0; j < dk; ++j) y[j] = J->dST ? J->dST[srow + j] : 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const size_t tok = tok0 + (size_t)t;
            const double *kt = J->k + tok * dk;
            const double *qt = J->q + tok * dk;
            const double *s0 = traj + (size_t)t * dk;
            const double *s1 = traj + (size_t)(t + 1) * dk;
            const double vi = J->v[tok * dv + i];
            const double g = J->dO ? J->dO[tok * dv + i] : 0.0;
            for (int j = 0; j < dk; ++j) {
                J->gq[tok * dk + j] += g * s1[j];
                y[j] += g * qt[j];
            }
            for (int j = 0; j < dk; ++j) x[j] = (diag ? J->alpha[tok * dk + j] : J->alpha[tok]) * s0[j];
            double yk = 0.0;
            for (int j = 0; j < dk; ++j) yk += y[j] * kt[j];
            if (delta) {
                const double be = J->beta[tok];
                const double bw = split ? J->beta[wplane + tok] : be;
                double p = 0.0;
                for (int j = 0; j < dk; ++j) p += x[j] * kt[j];
                J->gv[tok * dv + i] = bw * yk;
                if (split) {
                    J->gbeta[tok] -= yk * p;
                    J->gbeta[wplane + tok] += yk * vi;
                } else {
                    J->gbeta[tok] += yk * (vi - p);
                }
                for (int j = 0; j < dk; ++j) {
                    J->gk[tok * dk + j] += (bw * vi - be * p) * y[j] - be * yk * x[j];
                    dx[j] = y[j] - be * yk * kt[j];
                }
            } else {
                J->gv[tok * dv + i] = yk;
                for (int j = 0; j < dk; ++j) {
                    J->gk[tok * dk + j] += vi * y[j];
                    dx[j] = y[j];
                }
            }
            if (diag) {
                for (int j = 0; j < dk; ++j) J->galpha[tok * dk + j] += dx[j] * s0[j];
            } else {
                double acc = 0.0;
                for (int j = 0; j < dk; ++j) acc += dx[j] * s0[j];
                J->galpha[tok] += acc;
            }
            for (int j = 0; j < dk; ++j) y[j] = dx[j] * (diag ? J->alpha[tok * dk + j] : J->alpha[tok]);
        }
        for (int j = 0; j < dk; ++j) J->gS0[srow + j] = y[j];
    }
    free(traj); free(x); free(y); free(dx);
    return 0;
}

static void *bwd_worker(void *arg)
{
    bjob_t *J = (bjob_t *)arg;
    for (;;) {
        int64_t h = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (h >= J->BH) break;
        if (bwd_head(J, h) != 0) __atomic_store_n(&J->failed, 1, __ATOMIC_RELAXED);
    }
    return NULL;
}

/*
 * Gradients of L = sum <dO, o> + <dST, S_T> with respect to every input.
 *   q, k: [BH, T, dk]   v: [BH, T, dv]   alpha: [BH, T] ([BH, T, dk] in modes 3, 4)
 *   beta: [BH, T] (modes 0, 3; NULL in modes 1, 4; [2, BH, T] in mode 2: erase, then
 *         write strengths)   S0: [BH, dv, dk] or NULL (zero)
 *   dO: [BH, T, dv] or NULL (zero)   dST: [BH, dv, dk] or NULL (zero)
 *   outputs: gq, gk like q; gv like v; galpha like alpha; gbeta like beta (modes
 *   0, 2, 3; may be NULL otherwise); gS0 [BH, dv, dk].  All float64.
 * Returns the number of threads used, or -1 on bad arguments or allocation
 * failure.
 */
int oracle_scan_bwd_f64(int mode, int64_t BH, int64_t T, int dk, int dv,
                        const double *q, const double *k, const double *v,
                        const double *alpha, const double *beta, const double *S0,
                        const double *dO, const double *dST,
                        double *gq, double *gk, double *gv, double *galpha, double *gbeta,
                        double *gS0, int nthreads)
{
    if (mode < ORACLE_GDN || mode > ORACLE_GLA_DIAG) return -1;
    if (BH < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    const int delta = mode == ORACLE_GDN || mode == ORACLE_GDN_DIAG || mode == ORACLE_GDN_EW;
    if (BH * T > 0 && (!q || !k || !v || !alpha || !gq || !gk || !gv || !galpha)) return -1;
    if (delta && BH * T > 0 && (!beta || !gbeta)) return -1;
    if (BH > 0 && !gS0) return -1;
    if (nthreads < 1) nthreads = 1;
    bjob_t J;
    memset(&J, 0, sizeof J);
    J.mode = mode; J.BH = BH; J.T = T; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = delta ? beta : NULL; J.S0 = S0;
    J.dO = dO; J.dST = dST;
    J.gq = gq; J.gk = gk; J.gv = gv; J.galpha = galpha; J.gbeta = delta ? gbeta : NULL; J.gS0 = gS0;
    if (BH == 0) return 1;
    if ((int64_t)nthreads > BH) nthreads = (int)BH;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -1;
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, bwd_worker, &J) != 0) break;
        ++started;
    }
    bwd_worker(&J);
    for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    return J.failed ? -1 : started + 1;
}
