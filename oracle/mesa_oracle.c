/*
 * mesa_oracle.c -- plain, slow fp64 CPU reference of the Mesa layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no code with the HIP library.
 *
 * What it computes (MesaNet summary, gist.science paper 2506.05233):
 *  - Section "A Camada Mesa", displayed objective: Phi_t minimises
 *      1/2 sum_{t'<=t} zeta_{tt'} |v_t' - Phi k_t'|^2 + 1/2 Tr(Phi Lambda Phi^T).
 *    Setting its gradient to zero gives Phi_t (H_t + Lambda) = G_t with
 *      H_t = sum zeta_{tt'} k_t' k_t'^T   (d_k x d_k)
 *      G_t = sum zeta_{tt'} v_t' k_t'^T   (d_v x d_k).
 *    With zeta_{tt'} = prod_{s=t'+1..t} gamma_s ("cumulative forget
 *    factors") these obey H_t = gamma_t H_{t-1} + k_t k_t^T and
 *    G_t = gamma_t G_{t-1} + v_t k_t^T, H_0 = G_0 = 0.
 *  - Same section, sentence after the objective: the output is
 *    Delta_t = Phi_t q_t = G_t q*_t with q*_t = (H_t + Lambda)^{-1} q_t,
 *    the solve done by Conjugate Gradient.
 *  - Same section, bullet "Computacao Dinamica": the number of CG
 *    iterations needed to meet a stopping criterion varies per token.
 *
 * Readings where the page is silent (each one listed in the design notes):
 *  - Lambda = diag(lambda), one lambda vector per head, constant in t.
 *  - CG is the textbook unpreconditioned method started from x0 = 0.
 *  - Stopping: before each update, stop when |r|_2 / |q_t|_2 < tol, where r
 *    is the recursively updated residual; tol == 0 runs exactly max_iters
 *    updates.  rr == 0 or p^T A p <= 0 also stop (breakdown guards); q_t = 0
 *    gives x = 0 and zero iterations.
 *  - The output is G_t x_k, with x_k the CG iterate that was reached.
 *
 * The H_t and G_t are formed explicitly per token, in fp64, exactly as the
 * recurrence above says.  No chunking, no blocking.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    ORACLE_STOP_CAP = 0,       /* max_iters updates were made            */
    ORACLE_STOP_TOL = 1,       /* residual ratio fell below tol          */
    ORACLE_STOP_RR_ZERO = 2,   /* r^T r == 0 (exact convergence)         */
    ORACLE_STOP_BREAKDOWN = 3, /* p^T A p <= 0 (cannot occur for SPD A)  */
    ORACLE_STOP_Q_ZERO = 4     /* q_t == 0: x = 0                        */
};

static double dot(int n, const double *a, const double *b)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* y = (Hm + diag(lam)) p, Hm is n x n row-major. */
static void apply_a(int n, const double *Hm, const double *lam, const double *p, double *y)
{
    for (int i = 0; i < n; ++i) {
        double s = 0.0;
        for (int j = 0; j < n; ++j) s += Hm[(size_t)i * n + j] * p[j];
        y[i] = s + lam[i] * p[i];
    }
}

/*
 * Conjugate Gradient on (Hm + diag(lam)) x = b from x = x0 (x0 == NULL: from
 * x = 0, the page's solve; a given x0 is the warm start that the page names
 * as future work in "Significancia e Alegacoes").  From x0 the method is the
 * same with r0 = b - A x0 and p0 = r0.  The stop test always compares |r|
 * with |b|.  b == 0 gives x = 0 and no update, whatever x0 is.
 * Outputs: x, number of updates (return value), the stop reason, the residual
 * ratio rho at the stop (rho_n = sqrt(r^T r)/|b| after the last update) and
 * the smallest ratio that was checked and passed before it (+inf if none).
 * scratch: 3n doubles.  x may alias x0.
 */
int oracle_cg_solve_from(int n, const double *Hm, const double *lam, const double *b,
                         const double *x0, int max_iters, double tol, double *x, double *scratch,
                         int *reason, double *rho_stop, double *rho_min_prev)
{
    double *r = scratch, *p = scratch + n, *y = scratch + 2 * n;
    double nq = sqrt(dot(n, b, b));
    if (nq == 0.0) {
        for (int i = 0; i < n; ++i) x[i] = 0.0;
        if (reason) *reason = ORACLE_STOP_Q_ZERO;
        if (rho_stop) *rho_stop = 0.0;
        if (rho_min_prev) *rho_min_prev = INFINITY;
        return 0;
    }
    if (x0) {
        for (int i = 0; i < n; ++i) x[i] = x0[i];
        apply_a(n, Hm, lam, x, y);
        for (int i = 0; i < n; ++i) { r[i] = b[i] - y[i]; p[i] = r[i]; }
    } else {
        for (int i = 0; i < n; ++i) { x[i] = 0.0; r[i] = b[i]; p[i] = b[i]; }
    }
    double rr = dot(n, r, r);
    double minprev = INFINITY;
    int it = 0, why = ORACLE_STOP_CAP;
    while (it < max_iters) {
        double rho = sqrt(rr) / nq;
        if (tol > 0.0 && rho < tol) { why = ORACLE_STOP_TOL; break; }
        if (rr == 0.0) { why = ORACLE_STOP_RR_ZERO; break; }
        apply_a(n, Hm, lam, p, y);
        double pap = dot(n, p, y);
        if (!(pap > 0.0)) { why = ORACLE_STOP_BREAKDOWN; break; }
        double alpha = rr / pap;
        for (int i = 0; i < n; ++i) { x[i] += alpha * p[i]; r[i] -= alpha * y[i]; }
        double rr_new = dot(n, r, r);
        double beta = rr_new / rr;
        for (int i = 0; i < n; ++i) p[i] = r[i] + beta * p[i];
        rr = rr_new;
        if (rho < minprev) minprev = rho;
        ++it;
    }
    if (reason) *reason = why;
    if (rho_stop) *rho_stop = sqrt(rr) / nq;
    if (rho_min_prev) *rho_min_prev = minprev;
    return it;
}

/* The page's solve: CG from x = 0. */
int oracle_cg_solve(int n, const double *Hm, const double *lam, const double *b,
                    int max_iters, double tol, double *x, double *scratch,
                    int *reason, double *rho_stop, double *rho_min_prev)
{
    return oracle_cg_solve_from(n, Hm, lam, b, NULL, max_iters, tol, x, scratch, reason,
                                rho_stop, rho_min_prev);
}

/* H = g*H + a b^T  (rows x cols, row-major) */
static void decay_rank1(int rows, int cols, double *M, double g, const double *a, const double *b)
{
    for (int i = 0; i < rows; ++i)
        for (int j = 0; j < cols; ++j)
            M[(size_t)i * cols + j] = g * M[(size_t)i * cols + j] + a[i] * b[j];
}

/* out = M x  (rows x cols) */
static void matvec(int rows, int cols, const double *M, const double *x, double *out)
{
    for (int i = 0; i < rows; ++i) out[i] = dot(cols, M + (size_t)i * cols, x);
}

/*
 * One token of the recurrence plus its solve: update Hs, Gs in place with
 * (gamma, k, v), then CG on (Hs + diag lam) x = q and out = Gs x.
 */
static void token_step(int dk, int dv, double *Hs, double *Gs, double g,
                       const double *q, const double *k, const double *v,
                       const double *lam, int max_iters, double tol, int solve,
                       double *out, int *iters, double *rho_stop, double *rho_min_prev,
                       int *reason, double *x, double *scratch)
{
    decay_rank1(dk, dk, Hs, g, k, k);
    decay_rank1(dv, dk, Gs, g, v, k);
    if (!solve) return;
    int why = 0;
    double rs = 0.0, rm = 0.0;
    int n = oracle_cg_solve(dk, Hs, lam, q, max_iters, tol, x, scratch, &why, &rs, &rm);
    matvec(dv, dk, Gs, x, out);
    if (iters) *iters = n;
    if (rho_stop) *rho_stop = rs;
    if (rho_min_prev) *rho_min_prev = rm;
    if (reason) *reason = why;
}

/*
 * Forward pass over [B, H, T] tokens.
 *   q, k : [B,H,T,dk]   v : [B,H,T,dv]   gamma : [B,H,T]   lam : [H,dk]
 *   want : [B,H,T] bytes or NULL; a token with want == 0 still updates the
 *          state but is not solved (its outputs are left untouched).
 *   out  : [B,H,T,dv]; iters, reason : [B,H,T] int32; rho_stop,
 *          rho_min_prev : [B,H,T] (each may be NULL)
 *   final_H : [B,H,dk,dk], final_G : [B,H,dv,dk] or NULL.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_forward(const double *q, const double *k, const double *v,
                   const double *gamma, const double *lam,
                   int B, int H, int T, int dk, int dv, int max_iters, double tol,
                   const uint8_t *want, double *out, int32_t *iters,
                   double *rho_stop, double *rho_min_prev, int32_t *reason,
                   double *final_H, double *final_G)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0 || max_iters < 0 || !(tol >= 0.0))
        return -1;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long bh = 0; bh < (long)B * H; ++bh) {
        int h = (int)(bh % H);
        double *Hs = calloc((size_t)dk * dk, sizeof(double));
        double *Gs = calloc((size_t)dv * dk, sizeof(double));
        double *x = malloc(sizeof(double) * dk);
        double *scratch = malloc(sizeof(double) * 3 * dk);
        if (!Hs || !Gs || !x || !scratch) {
            bad = 1;
        } else {
            for (int t = 0; t < T; ++t) {
                size_t tok = (size_t)bh * T + t;
                int solve = want ? want[tok] != 0 : 1;
                int it = 0, why = 0;
                double rs = 0.0, rm = 0.0;
                token_step(dk, dv, Hs, Gs, gamma[tok], q + tok * dk, k + tok * dk,
                           v + tok * dv, lam + (size_t)h * dk, max_iters, tol, solve,
                           out + tok * dv, &it, &rs, &rm, &why, x, scratch);
                if (solve) {
                    if (iters) iters[tok] = it;
                    if (rho_stop) rho_stop[tok] = rs;
                    if (rho_min_prev) rho_min_prev[tok] = rm;
                    if (reason) reason[tok] = why;
                }
            }
            if (final_H) memcpy(final_H + (size_t)bh * dk * dk, Hs, sizeof(double) * dk * dk);
            if (final_G) memcpy(final_G + (size_t)bh * dv * dk, Gs, sizeof(double) * dv * dk);
        }
        free(Hs); free(Gs); free(x); free(scratch);
    }
    return bad ? -1 : 0;
}

/*
 * One recurrent decode step for N x H heads (same section, bullet
 * "Paralelizacao": O(1) inference with the states G_t, H_t).
 *   q, k : [N,H,dk]  v : [N,H,dv]  gamma : [N,H]  lam : [H,dk]
 *   state_H : [N,H,dk,dk], state_G : [N,H,dv,dk] (updated in place)
 *   out : [N,H,dv]; iters, reason : [N,H]; rho_stop, rho_min_prev : [N,H]
 */
int oracle_decode_step(const double *q, const double *k, const double *v,
                       const double *gamma, const double *lam,
                       double *state_H, double *state_G,
                       int N, int H, int dk, int dv, int max_iters, double tol,
                       double *out, int32_t *iters, double *rho_stop,
                       double *rho_min_prev, int32_t *reason)
{
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0 || max_iters < 0 || !(tol >= 0.0))
        return -1;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long nh = 0; nh < (long)N * H; ++nh) {
        int h = (int)(nh % H);
        double *x = malloc(sizeof(double) * dk);
        double *scratch = malloc(sizeof(double) * 3 * dk);
        if (!x || !scratch) {
            bad = 1;
        } else {
            int it = 0, why = 0;
            double rs = 0.0, rm = 0.0;
            token_step(dk, dv, state_H + (size_t)nh * dk * dk, state_G + (size_t)nh * dv * dk,
                       gamma[nh], q + (size_t)nh * dk, k + (size_t)nh * dk, v + (size_t)nh * dv,
                       lam + (size_t)h * dk, max_iters, tol, 1, out + (size_t)nh * dv,
                       &it, &rs, &rm, &why, x, scratch);
            if (iters) iters[nh] = it;
            if (rho_stop) rho_stop[nh] = rs;
            if (rho_min_prev) rho_min_prev[nh] = rm;
            if (reason) reason[nh] = why;
        }
        free(x); free(scratch);
    }
    return bad ? -1 : 0;
}

/*
 * One decode step with a warm-started solve (the warm start that the page
 * names as future work, section "Significancia e Alegacoes"), for N x H heads.
 * Same as oracle_decode_step, plus state_x [N,H,dk]: on entry the previous
 * step's solution of each head, on exit this step's.  The start point is
 *   mode 0: x0 = 0 (the page's cold start);
 *   mode 1: x0 = x_prev;
 *   mode 2: x0 = c x_prev with c = (x_prev . q) / (x_prev . A x_prev), the
 *           minimiser of the A-norm error over multiples of x_prev (x0 = 0
 *           when x_prev . A x_prev <= 0, e.g. x_prev = 0).
 */
int oracle_decode_step_warm(const double *q, const double *k, const double *v,
                            const double *gamma, const double *lam,
                            double *state_H, double *state_G, double *state_x,
                            int N, int H, int dk, int dv, int max_iters, double tol, int mode,
                            double *out, int32_t *iters, double *rho_stop,
                            double *rho_min_prev, int32_t *reason)
{
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0 || max_iters < 0 || !(tol >= 0.0) ||
        mode < 0 || mode > 2)
        return -1;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long nh = 0; nh < (long)N * H; ++nh) {
        int h = (int)(nh % H);
        double *x0 = malloc(sizeof(double) * dk);
        double *ax = malloc(sizeof(double) * dk);
        double *scratch = malloc(sizeof(double) * 3 * dk);
        if (!x0 || !ax || !scratch) {
            bad = 1;
        } else {
            double *Hs = state_H + (size_t)nh * dk * dk, *Gs = state_G + (size_t)nh * dv * dk;
            double *xs = state_x + (size_t)nh * dk;
            const double *qh = q + (size_t)nh * dk, *lh = lam + (size_t)h * dk;
            decay_rank1(dk, dk, Hs, gamma[nh], k + (size_t)nh * dk, k + (size_t)nh * dk);
            decay_rank1(dv, dk, Gs, gamma[nh], v + (size_t)nh * dv, k + (size_t)nh * dk);
            double c = 0.0;
            if (mode == 1) {
                c = 1.0;
            } else if (mode == 2) {
                apply_a(dk, Hs, lh, xs, ax);
                double den = dot(dk, xs, ax);
                c = den > 0.0 ? dot(dk, xs, qh) / den : 0.0;
            }
            for (int i = 0; i < dk; ++i) x0[i] = c * xs[i];
            int why = 0;
            double rs = 0.0, rm = 0.0;
            int it = oracle_cg_solve_from(dk, Hs, lh, qh, mode == 0 ? NULL : x0, max_iters, tol,
                                          xs, scratch, &why, &rs, &rm);
            matvec(dv, dk, Gs, xs, out + (size_t)nh * dv);
            if (iters) iters[nh] = it;
            if (rho_stop) rho_stop[nh] = rs;
            if (rho_min_prev) rho_min_prev[nh] = rm;
            if (reason) reason[nh] = why;
        }
        free(x0); free(ax); free(scratch);
    }
    return bad ? -1 : 0;
}

/*
 * Query/key pre-processing before the layer (MesaNet summary, section
 * "Arquitetura (MesaNet)", bullet "Pre-processamento": keys and queries are
 * normalised and convolved with a small window before the Mesa layer).
 * Reading: a causal depthwise convolution over the token axis, per head and
 * feature, of width W, followed by L2 normalisation of each token's vector:
 *   c_t[f] = sum_{j=0..W-1} w[h][j][f] x_{t-j}[f]
 *   y_t    = c_t / |c_t|_2        (y_t = 0 when c_t = 0)
 * Rows before t = 0 come from hist ([B,H,W-1,d], oldest first; NULL = zeros),
 * so a sequence can be processed in pieces.  hist_out (may be NULL) receives
 * the last W-1 input rows of hist followed by x, for the next piece.
 *   x : [B,H,T,d]   w : [H,W,d]   y : [B,H,T,d]
 */
int oracle_qk_preprocess(const double *x, const double *w, int W, const double *hist,
                         double *hist_out, int B, int H, int T, int d, double *y)
{
    if (B < 0 || H < 0 || T < 0 || d <= 0 || W < 1) return -1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < (long)B * H; ++bh) {
        int h = (int)(bh % H);
        const double *xb = x + (size_t)bh * T * d;
        const double *hb = hist ? hist + (size_t)bh * (W - 1) * d : NULL;
        for (int t = 0; t < T; ++t) {
            double *yt = y + ((size_t)bh * T + t) * d;
            double ss = 0.0;
            for (int f = 0; f < d; ++f) {
                double c = 0.0;
                for (int j = 0; j < W; ++j) {
                    int src = t - j;           /* token index; < 0 reaches into hist */
                    double xv;
                    if (src >= 0) xv = xb[(size_t)src * d + f];
                    else xv = hb ? hb[(size_t)(W - 1 + src) * d + f] : 0.0;
                    c += w[((size_t)h * W + j) * d + f] * xv;
                }
                yt[f] = c;
                ss += c * c;
            }
            double nrm = sqrt(ss);
            for (int f = 0; f < d; ++f) yt[f] = nrm > 0.0 ? yt[f] / nrm : 0.0;
        }
        if (hist_out) {
            double *ho = hist_out + (size_t)bh * (W - 1) * d;
            for (int r = 0; r < W - 1; ++r) {
                int src = T - (W - 1) + r;     /* position in x; < 0 reaches into hist */
                for (int f = 0; f < d; ++f) {
                    double xv;
                    if (src >= 0) xv = xb[(size_t)src * d + f];
                    else xv = hb ? hb[(size_t)(W - 1 + src) * d + f] : 0.0;
                    ho[(size_t)r * d + f] = xv;
                }
            }
        }
    }
    return 0;
}

/*
 * Backward pass of the layer for a loss L with dL/do_t = gout_t.  The page
 * says the layer trains in parallel but gives no gradient (section "A Camada
 * Mesa", bullet "Paralelizacao").  Reading: differentiate o_t = G_t A_t^{-1}
 * q_t (A_t = H_t + Lambda) implicitly, evaluated at the CG solutions, with
 * the adjoint solve done by the same k-step CG:
 *   x_t  = CG(A_t, q_t)                (the forward's solution)
 *   bx_t = G_t^T gout_t,   z_t = CG(A_t, bx_t)
 *   dL/dq_t      = z_t
 *   dL/dG_t      = gout_t x_t^T,      dL/dH_t = -z_t x_t^T
 *   dL/dlambda   = -sum_t z_t (.) x_t            (summed over the batch)
 *   dL/dv_i      = sum_{t>=i} zeta_ti (x_t . k_i) gout_t
 *   dL/dk_i      = sum_{t>=i} zeta_ti [(gout_t . v_i) x_t - (x_t . k_i) z_t - (z_t . k_i) x_t]
 *   dL/dln gamma_s = sum_{t>=s} (beta_t - a_t), with
 *     beta_t = gout_t . (G_t x_t) - z_t . (H_t x_t)
 *     a_i    = (v_i . dL/dv_i + k_i . dL/dk_i) / 2
 *   (the sum over pairs i < s <= t of zeta_ti (k_i . x_t)[(gout_t . v_i) - (z_t . k_i)],
 *   split into its query-side and key-side totals), and dL/dgamma_s =
 *   dL/dln gamma_s / gamma_s.  The key-side sums run backwards over t with the
 *   states P_gx = sum_{t>=i} zeta_ti gout_t x_t^T and P_zx = sum zeta_ti z_t x_t^T.
 * Shapes as oracle_forward; gout [B,H,T,dv]; dq, dk [B,H,T,dk]; dv [B,H,T,dv];
 * dgamma [B,H,T]; dlam [H,dk]; x_out [B,H,T,dk] and the adjoint solve's
 * z_iters / z_rho_stop / z_rho_min_prev / z_reason [B,H,T] may be NULL.
 */
int oracle_backward(const double *q, const double *k, const double *v, const double *gamma,
                    const double *lam, const double *gout, int B, int H, int T, int dk, int dv,
                    int max_iters, double tol, double *x_out, double *dq, double *dk_out,
                    double *dv_out, double *dgamma, double *dlam, int32_t *z_iters,
                    double *z_rho_stop, double *z_rho_min_prev, int32_t *z_reason)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0 || max_iters < 0 || !(tol >= 0.0))
        return -1;
    double *part = calloc((size_t)B * H * dk + 1, sizeof(double));   /* per-(b,h) dlambda */
    if (!part) return -1;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long bh = 0; bh < (long)B * H; ++bh) {
        int h = (int)(bh % H);
        const double *lh = lam + (size_t)h * dk;
        double *Hs = calloc((size_t)dk * dk, sizeof(double));
        double *Gs = calloc((size_t)dv * dk, sizeof(double));
        double *X = malloc(sizeof(double) * ((size_t)T * dk + 1));
        double *Z = malloc(sizeof(double) * ((size_t)T * dk + 1));
        double *beta = malloc(sizeof(double) * ((size_t)T + 1));
        double *o = malloc(sizeof(double) * dv);
        double *bx = malloc(sizeof(double) * dk);
        double *c = malloc(sizeof(double) * dk);
        double *scratch = malloc(sizeof(double) * 3 * dk);
        double *Pgx = calloc((size_t)dv * dk, sizeof(double));
        double *Pzx = calloc((size_t)dk * dk, sizeof(double));
        if (!Hs || !Gs || !X || !Z || !beta || !o || !bx || !c || !scratch || !Pgx || !Pzx) {
            bad = 1;
        } else {
            /* forward sweep: states, x_t, the adjoint solve z_t, beta_t, dlambda */
            for (int t = 0; t < T; ++t) {
                size_t tok = (size_t)bh * T + t;
                const double *kt = k + tok * dk, *vt = v + tok * dv, *gt = gout + tok * dv;
                decay_rank1(dk, dk, Hs, gamma[tok], kt, kt);
                decay_rank1(dv, dk, Gs, gamma[tok], vt, kt);
                double *xt = X + (size_t)t * dk, *zt = Z + (size_t)t * dk;
                oracle_cg_solve(dk, Hs, lh, q + tok * dk, max_iters, tol, xt, scratch, NULL, NULL, NULL);
                matvec(dv, dk, Gs, xt, o);
                for (int f = 0; f < dk; ++f) {
                    double s = 0.0;
                    for (int i = 0; i < dv; ++i) s += Gs[(size_t)i * dk + f] * gt[i];
                    bx[f] = s;
                }
                int why = 0;
                double rs = 0.0, rm = 0.0;
                int it = oracle_cg_solve(dk, Hs, lh, bx, max_iters, tol, zt, scratch, &why, &rs, &rm);
                if (z_iters) z_iters[tok] = it;
                if (z_rho_stop) z_rho_stop[tok] = rs;
                if (z_rho_min_prev) z_rho_min_prev[tok] = rm;
                if (z_reason) z_reason[tok] = why;
                matvec(dk, dk, Hs, xt, c);
                beta[t] = dot(dv, gt, o) - dot(dk, zt, c);
                for (int f = 0; f < dk; ++f) part[(size_t)bh * dk + f] -= zt[f] * xt[f];
                if (x_out) memcpy(x_out + tok * dk, xt, sizeof(double) * dk);
                memcpy(dq + tok * dk, zt, sizeof(double) * dk);
            }
            /* reverse sweep: key-side sums, then the log-gate gradient */
            double acc = 0.0;
            for (int t = T - 1; t >= 0; --t) {
                size_t tok = (size_t)bh * T + t;
                const double *kt = k + tok * dk, *vt = v + tok * dv, *gt = gout + tok * dv;
                const double *xt = X + (size_t)t * dk, *zt = Z + (size_t)t * dk;
                double gnext = (t + 1 < T) ? gamma[tok + 1] : 0.0;
                decay_rank1(dv, dk, Pgx, gnext, gt, xt);
                decay_rank1(dk, dk, Pzx, gnext, zt, xt);
                double *dvt = dv_out + tok * dv, *dkt = dk_out + tok * dk;
                matvec(dv, dk, Pgx, kt, dvt);
                for (int f = 0; f < dk; ++f) {
                    double s = 0.0;
                    for (int i = 0; i < dv; ++i) s += Pgx[(size_t)i * dk + f] * vt[i];
                    for (int e = 0; e < dk; ++e)
                        s -= (Pzx[(size_t)f * dk + e] + Pzx[(size_t)e * dk + f]) * kt[e];
                    dkt[f] = s;
                }
                double a = 0.5 * (dot(dv, vt, dvt) + dot(dk, kt, dkt));
                acc += beta[t] - a;
                dgamma[tok] = acc / gamma[tok];
            }
        }
        free(Hs); free(Gs); free(X); free(Z); free(beta); free(o); free(bx); free(c);
        free(scratch); free(Pgx); free(Pzx);
    }
    if (!bad) {
        for (long i = 0; i < (long)H * dk; ++i) dlam[i] = 0.0;
        for (long bh = 0; bh < (long)B * H; ++bh)   /* fixed order over the batch */
            for (int f = 0; f < dk; ++f) dlam[(bh % H) * dk + f] += part[(size_t)bh * dk + f];
    }
    free(part);
    return bad ? -1 : 0;
}

/*
 * Recurrence of the Hawk layer that the hybrid "Hawk-Mesa" model alternates
 * with Mesa layers (section "Arquitetura (MesaNet)", bullet "Variante
 * Hibrida": LRU (Hawk) layers).  The page names the layer only; the reading
 * is the published real-gated linear recurrent unit of Hawk, per channel d:
 *   r_t = sigmoid(ga_t),  i_t = sigmoid(gx_t)        (gate pre-activations)
 *   log a_t = -c * softplus(-lam_d) * r_t            (a = sigmoid(lam), a_t = a^{c r_t})
 *   h_t = a_t h_{t-1} + sqrt(1 - a_t^2) * (i_t * x_t),  h_0 from h0 (NULL: 0)
 * x, ga, gx, y: [B, T, D]; lam: [D]; h0, h_final: [B, D] (may be NULL).
 */
static double softplus(double z) { return z > 30.0 ? z : log1p(exp(z)); }
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

int oracle_hawk_scan(const double *x, const double *ga, const double *gx, const double *lam, double c,
                     const double *h0, int B, int T, int D, double *y, double *h_final)
{
    if (B < 0 || T < 0 || D <= 0) return -1;
    #pragma omp parallel for schedule(static)
    for (long bd = 0; bd < (long)B * D; ++bd) {
        long b = bd / D;
        int d = (int)(bd % D);
        double h = h0 ? h0[bd] : 0.0;
        double sp = softplus(-lam[d]);
        for (int t = 0; t < T; ++t) {
            size_t i = ((size_t)b * T + t) * D + d;
            double r = sigmoid(ga[i]), in = sigmoid(gx[i]);
            double a = exp(-c * sp * r);
            h = a * h + sqrt(1.0 - a * a) * (in * x[i]);
            y[i] = h;
        }
        if (h_final) h_final[bd] = h;
    }
    return 0;
}

/* Threads an OpenMP parallel region of this library would use. */
int oracle_max_threads(void) { return omp_get_max_threads(); }
