/*
 * gato_oracle.c -- plain, slow, fp64 CPU oracle for one SQP iteration's
 * linear-algebra core over a batch of independent LQ subproblems.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or helper with the HIP library: every routine below is written out
 * again from the definitions, in double precision, with plain loops.
 *
 * What it computes follows "GATO: GPU-Accelerated and Batched Trajectory
 * Optimization for Scalable Edge Model Predictive Control" (arXiv 2510.07625):
 *   Sec. II  -- the QP of Step 1 (eq. 1), its KKT system (eq. 2), the Schur
 *              complement S, gamma and the symmetric stair preconditioner
 *              (eqs. 4-6), PCG on S lambda = gamma, and the L1 merit (eq. 3);
 *   Sec. III -- the line search over step sizes (eq. 7).
 * The displayed equations are absent from the page text we have, so the
 * formulas are the textbook range-space (Schur-complement) method for the
 * equality-constrained QP that the surrounding prose describes.  Every
 * reading taken where the text is silent is named at the function doing it.
 * One of them is parity unpinned against the pages: the form of the stair
 * preconditioner, which the paper cites but does not print (its closed form,
 * symmetry and definiteness under the reading are pinned; only the PCG
 * iteration counts depend on it, not lambda or dz beyond the exit tolerance).
 *
 * Problem data, per solve b (N knot points, n states, m controls):
 *   Q[k] n x n (k < N), q[k] n, R[k] m x m (k < N-1), r[k] m,
 *   A[k] n x n, Bu[k] n x m, e[k] n (k < N-1), x0 n, rho (scalar damping).
 * The QP (reading of eq. 1, with e_k = f(x_k,u_k,h) - x_{k+1} as Sec. II
 * defines it):
 *   min  sum_k 1/2 dx_k'(Q_k + rho I)dx_k + q_k'dx_k
 *      + sum_{k<N-1} 1/2 du_k' R_k du_k + r_k'du_k
 *   s.t. dx_0 = x0,  dx_{k+1} = A_k dx_k + B_k du_k + e_k.
 * In block form: G dz = blkdiag(Q~_0, R_0, Q~_1, ..., Q~_{N-1}),
 * C dz = c with block row 0 = [I], block row k+1 = [-A_k, -B_k, I],
 * c = (x0, e_0, ..., e_{N-2}).  The KKT system (eq. 2) is
 *   G dz - C' lambda = -g,   C dz = c,
 * hence S = C G^-1 C', gamma = c + C G^-1 g, dz = G^-1 (C' lambda - g).
 *
 * Layouts (row-major, batch-major, unpadded):
 *   S, Pinv  [B][N][3][n][n]   block row k = [X_{k,k-1}, X_{k,k}, X_{k,k+1}],
 *                              out-of-range blocks are zero;
 *   gamma, lambda [B][N][n];  Qinv [B][N][n][n];  Rinv [B][N-1][m][m];
 *   dz [B][N*n + (N-1)*m] ordered dx_0, du_0, dx_1, ..., du_{N-2}, dx_{N-1}
 *   (the ordering dz_k = [dx_k du_k], dz_N = dx_N that Sec. II states).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define REF_F_Q_NOT_SPD 1
#define REF_F_R_NOT_SPD 2
#define REF_F_S_NOT_SPD 4
#define REF_F_PCG_MAXITER 8
#define REF_F_PCG_BREAKDOWN 16
#define REF_F_LS_FAILED 32
#define REF_F_NONFINITE 64

typedef struct {
    int n, m, N, B;
} gato_ref_dims;

/* ------------------------------------------------------------------ */
/* small dense helpers (row-major, plain loops)                       */
/* ------------------------------------------------------------------ */

/* C = A * B, A is r x s, B is s x t. */
static void mm(int r, int s, int t, const double* A, const double* B, double* C)
{
    for (int i = 0; i < r; ++i)
        for (int j = 0; j < t; ++j) {
            double acc = 0.0;
            for (int l = 0; l < s; ++l) acc += A[i * s + l] * B[l * t + j];
            C[i * t + j] = acc;
        }
}

/* C = A * B', A is r x s, B is t x s. */
static void mmT(int r, int s, int t, const double* A, const double* B, double* C)
{
    for (int i = 0; i < r; ++i)
        for (int j = 0; j < t; ++j) {
            double acc = 0.0;
            for (int l = 0; l < s; ++l) acc += A[i * s + l] * B[j * s + l];
            C[i * t + j] = acc;
        }
}

/* y = A x, A is r x s. */
static void mv(int r, int s, const double* A, const double* x, double* y)
{
    for (int i = 0; i < r; ++i) {
        double acc = 0.0;
        for (int l = 0; l < s; ++l) acc += A[i * s + l] * x[l];
        y[i] = acc;
    }
}

/* y = A' x, A is r x s (so y has s entries). */
static void mtv(int r, int s, const double* A, const double* x, double* y)
{
    for (int j = 0; j < s; ++j) {
        double acc = 0.0;
        for (int i = 0; i < r; ++i) acc += A[i * s + j] * x[i];
        y[j] = acc;
    }
}

/*
 * Inverse of a symmetric positive definite p x p matrix M through its
 * Cholesky factor M = L L'.  Returns 0 on success and 1 when a pivot is not
 * positive (or not finite): the matrix is then not SPD.  On failure the
 * output is still written (NaN where the factor broke down), so that a
 * flagged solve keeps running, as the Branch page's test protocol does for a
 * failed pivot: flagged, not repaired.
 */
static int spd_inverse(int p, const double* M, double* Minv)
{
    double* L = (double*)calloc((size_t)p * p, sizeof(double));
    double* Y = (double*)calloc((size_t)p * p, sizeof(double));
    int bad = 0;
    for (int j = 0; j < p; ++j) {
        double d = M[j * p + j];
        for (int l = 0; l < j; ++l) d -= L[j * p + l] * L[j * p + l];
        if (!(d > 0.0) || !isfinite(d)) bad = 1;
        double ljj = sqrt(d); /* NaN when d <= 0: the failure propagates */
        L[j * p + j] = ljj;
        for (int i = j + 1; i < p; ++i) {
            double s = M[i * p + j];
            for (int l = 0; l < j; ++l) s -= L[i * p + l] * L[j * p + l];
            L[i * p + j] = s / ljj;
        }
    }
    /* Solve L Y = I (forward substitution, column by column). */
    for (int c = 0; c < p; ++c)
        for (int i = 0; i < p; ++i) {
            double s = (i == c) ? 1.0 : 0.0;
            for (int l = 0; l < i; ++l) s -= L[i * p + l] * Y[l * p + c];
            Y[i * p + c] = s / L[i * p + i];
        }
    /* M^-1 = L^-T L^-1 = Y' Y. */
    for (int i = 0; i < p; ++i)
        for (int j = 0; j < p; ++j) {
            double s = 0.0;
            for (int l = 0; l < p; ++l) s += Y[l * p + i] * Y[l * p + j];
            Minv[i * p + j] = s;
        }
    free(L);
    free(Y);
    return bad;
}

/* ------------------------------------------------------------------ */
/* Stage 1: S, gamma, Phi^-1 (GATO paper Sec. II, eqs. 4-6)            */
/* ------------------------------------------------------------------ */

/*
 * Per solve: the inverses of the damped state-cost blocks Q~_k = Q_k + rho I
 * and of R_k (the G^-1 blocks of eq. 4), then the Schur complement blocks
 *   D_0     = Q~_0^-1,
 *   D_{k+1} = A_k Q~_k^-1 A_k' + B_k R_k^-1 B_k' + Q~_{k+1}^-1,
 *   S_{k,k+1} = -Q~_k^-1 A_k',   S_{k+1,k} = -A_k Q~_k^-1,
 * and the right-hand side
 *   gamma_0     = x0 + Q~_0^-1 q_0,
 *   gamma_{k+1} = e_k - A_k Q~_k^-1 q_k - B_k R_k^-1 r_k + Q~_{k+1}^-1 q_{k+1},
 * i.e. S = C G^-1 C' and gamma = c + C G^-1 g written out block by block
 * (reading of eqs. 4-6; theta_k, phi_k, zeta_k of eq. 5 are read as D_k,
 * S_{k+1,k} and G^-1 g).  The damping rho is added to the diagonal of Q_k as
 * the paper's hyper-parameter case study (Sec. IV-C) describes.
 *
 * Symmetric stair preconditioner (eq. 6; the paper cites it as its ref. [7]
 * and does not print it -- this is the reading used): with D = blkdiag(D_k),
 *   Phi^-1_{k,k}   = D_k^-1,
 *   Phi^-1_{k,k+1} = -D_k^-1 S_{k,k+1} D_{k+1}^-1,
 *   Phi^-1_{k+1,k} = -D_{k+1}^-1 S_{k+1,k} D_k^-1,
 * which is block-tridiagonal and symmetric (it equals D^-1 J S J D^-1 with
 * J = blkdiag((-1)^k I), hence SPD when S is).  Finalising the off-diagonal
 * blocks needs the neighbouring knot's D^-1, which is the one grid-wide
 * synchronisation the paper's setup kernel performs (Sec. III).
 */
static void form_one(const gato_ref_dims* d, int b, const double* Q, const double* q,
                     const double* R, const double* r, const double* A, const double* Bu,
                     const double* e, const double* x0, const double* rho, double* S,
                     double* Pinv, double* gamma, double* Qinv, double* Rinv, int* flags)
{
    const int n = d->n, m = d->m, N = d->N;
    const size_t nn = (size_t)n * n, mm_ = (size_t)m * m, nm = (size_t)n * m;
    const double* Qb = Q + (size_t)b * N * nn;
    const double* qb = q + (size_t)b * N * n;
    const double* Rb = R + (size_t)b * (N - 1) * mm_;
    const double* rb = r + (size_t)b * (N - 1) * m;
    const double* Ab = A + (size_t)b * (N - 1) * nn;
    const double* Bb = Bu + (size_t)b * (N - 1) * nm;
    const double* eb = e + (size_t)b * (N - 1) * n;
    const double* x0b = x0 + (size_t)b * n;
    double* Sb = S + (size_t)b * N * 3 * nn;
    double* Pb = Pinv + (size_t)b * N * 3 * nn;
    double* gb = gamma + (size_t)b * N * n;
    double* Qib = Qinv + (size_t)b * N * nn;
    double* Rib = Rinv + (size_t)b * (N - 1) * mm_;
    const double rh = rho ? rho[b] : 0.0;
    int fl = 0;

    double* Qt = (double*)malloc(nn * sizeof(double));
    double* W = (double*)malloc(nn * sizeof(double));
    double* T1 = (double*)malloc(nn * sizeof(double));
    double* V = (double*)malloc(nm * sizeof(double));
    double* T2 = (double*)malloc(nn * sizeof(double));
    double* Dinv = (double*)malloc((size_t)N * nn * sizeof(double));
    double* tv = (double*)malloc((size_t)(n > m ? n : m) * sizeof(double));
    double* tv2 = (double*)malloc((size_t)(n > m ? n : m) * sizeof(double));

    memset(Sb, 0, (size_t)N * 3 * nn * sizeof(double));
    memset(Pb, 0, (size_t)N * 3 * nn * sizeof(double));

    /* G^-1 blocks. */
    for (int k = 0; k < N; ++k) {
        for (size_t i = 0; i < nn; ++i) Qt[i] = Qb[k * nn + i];
        for (int i = 0; i < n; ++i) Qt[i * n + i] += rh;
        if (spd_inverse(n, Qt, Qib + k * nn)) fl |= REF_F_Q_NOT_SPD;
    }
    for (int k = 0; k < N - 1; ++k)
        if (spd_inverse(m, Rb + k * mm_, Rib + k * mm_)) fl |= REF_F_R_NOT_SPD;

    /* Diagonal blocks D_k and gamma_k: the own-knot terms first. */
    for (int k = 0; k < N; ++k) {
        double* Dk = Sb + ((size_t)k * 3 + 1) * nn;
        for (size_t i = 0; i < nn; ++i) Dk[i] = Qib[k * nn + i];
        mv(n, n, Qib + k * nn, qb + (size_t)k * n, gb + (size_t)k * n);
    }
    for (int i = 0; i < n; ++i) gb[i] += x0b[i];

    /* Coupling terms from knot k into knot k+1. */
    for (int k = 0; k < N - 1; ++k) {
        const double* Ak = Ab + k * nn;
        const double* Bk = Bb + k * nm;
        const double* Qik = Qib + k * nn;
        const double* Rik = Rib + k * mm_;
        mm(n, n, n, Ak, Qik, W);     /* W = A_k Q~_k^-1 */
        mmT(n, n, n, W, Ak, T1);     /* A_k Q~_k^-1 A_k' */
        mm(n, m, m, Bk, Rik, V);     /* V = B_k R_k^-1 */
        mmT(n, m, n, V, Bk, T2);     /* B_k R_k^-1 B_k' */
        double* Dk1 = Sb + ((size_t)(k + 1) * 3 + 1) * nn;
        for (size_t i = 0; i < nn; ++i) Dk1[i] += T1[i] + T2[i];
        /* S_{k+1,k} = -A_k Q~_k^-1 and S_{k,k+1} = its transpose. */
        double* Slo = Sb + ((size_t)(k + 1) * 3 + 0) * nn;
        double* Sup = Sb + ((size_t)k * 3 + 2) * nn;
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) {
                Slo[i * n + j] = -W[i * n + j];
                Sup[j * n + i] = -W[i * n + j];
            }
        /* gamma_{k+1} += e_k - A_k Q~_k^-1 q_k - B_k R_k^-1 r_k */
        mv(n, n, W, qb + (size_t)k * n, tv);
        mv(n, m, V, rb + (size_t)k * m, tv2);
        double* gk1 = gb + (size_t)(k + 1) * n;
        for (int i = 0; i < n; ++i) gk1[i] += eb[(size_t)k * n + i] - tv[i] - tv2[i];
    }

    /* Preconditioner: D_k^-1, then the off-diagonal stair blocks. */
    for (int k = 0; k < N; ++k) {
        const double* Dk = Sb + ((size_t)k * 3 + 1) * nn;
        if (spd_inverse(n, Dk, Dinv + k * nn)) fl |= REF_F_S_NOT_SPD;
        double* Pd = Pb + ((size_t)k * 3 + 1) * nn;
        for (size_t i = 0; i < nn; ++i) Pd[i] = Dinv[k * nn + i];
    }
    for (int k = 0; k < N - 1; ++k) {
        const double* Sup = Sb + ((size_t)k * 3 + 2) * nn;
        const double* Slo = Sb + ((size_t)(k + 1) * 3 + 0) * nn;
        double* Pup = Pb + ((size_t)k * 3 + 2) * nn;
        double* Plo = Pb + ((size_t)(k + 1) * 3 + 0) * nn;
        mm(n, n, n, Dinv + k * nn, Sup, T1);           /* D_k^-1 S_{k,k+1} */
        mm(n, n, n, T1, Dinv + (size_t)(k + 1) * nn, T2);
        for (size_t i = 0; i < nn; ++i) Pup[i] = -T2[i];
        mm(n, n, n, Dinv + (size_t)(k + 1) * nn, Slo, T1); /* D_{k+1}^-1 S_{k+1,k} */
        mm(n, n, n, T1, Dinv + k * nn, T2);
        for (size_t i = 0; i < nn; ++i) Plo[i] = -T2[i];
    }
    flags[b] = fl;
    free(Qt); free(W); free(T1); free(V); free(T2); free(Dinv); free(tv); free(tv2);
}

int gato_ref_form_schur(const gato_ref_dims* d, const double* Q, const double* q, const double* R,
                        const double* r, const double* A, const double* Bu, const double* e,
                        const double* x0, const double* rho, double* S, double* Pinv,
                        double* gamma, double* Qinv, double* Rinv, int* flags)
{
    if (!d || d->n < 1 || d->m < 1 || d->N < 1 || d->B < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < d->B; ++b)
        form_one(d, b, Q, q, R, r, A, Bu, e, x0, rho, S, Pinv, gamma, Qinv, Rinv, flags);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Stage 2: PCG on S lambda = gamma, then dz (GATO paper Sec. II)      */
/* ------------------------------------------------------------------ */

/* y = X v for a block-tridiagonal X stored as block rows [N][3][n][n]. */
static void btd_mv(int n, int N, const double* X, const double* v, double* y)
{
    const size_t nn = (size_t)n * n;
    for (int k = 0; k < N; ++k)
        for (int i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int s = 0; s < 3; ++s) {
                int kk = k + s - 1;
                if (kk < 0 || kk >= N) continue;
                const double* blk = X + ((size_t)k * 3 + s) * nn;
                for (int j = 0; j < n; ++j) acc += blk[i * n + j] * v[(size_t)kk * n + j];
            }
            y[(size_t)k * n + i] = acc;
        }
}

static double dot(size_t len, const double* a, const double* b)
{
    double s = 0.0;
    for (size_t i = 0; i < len; ++i) s += a[i] * b[i];
    return s;
}

/*
 * Preconditioned conjugate gradient on S lambda = gamma with the stair
 * preconditioner Phi^-1 (GATO paper Sec. II: iterate to tolerance eps using
 * products with S and Phi^-1 and vector reductions).  Starting point lambda
 * as given (the caller's warm start, zero by default).  Each iteration:
 *   v = S p;  a = eta / p'v;  lambda += a p;  r -= a v;
 *   stop when ||r||_2 <= eps ||gamma||_2 (the recurred residual: reading of
 *   "up to tolerance eps" as a relative residual test after the r update);
 *   z = Phi^-1 r;  eta' = r'z;  p = z + (eta'/eta) p.
 * The iteration count is the number of products with S inside the loop.
 * Flags: p'Sp <= 0 -> breakdown; a non-finite reduction -> nonfinite;
 * max_iters reached without meeting the test -> maxiter (the GATO docs'
 * max_pcg_iters cap).  ||gamma|| = 0 returns lambda = 0 after 0 iterations.
 */
static void pcg_one(const gato_ref_dims* d, int b, const double* S, const double* Pinv,
                    const double* gamma, double eps, int max_iters, double* lambda,
                    int* iters, double* relres, int* flags)
{
    const int n = d->n, N = d->N;
    const size_t len = (size_t)N * n;
    const size_t nn = (size_t)n * n;
    const double* Sb = S + (size_t)b * N * 3 * nn;
    const double* Pb = Pinv + (size_t)b * N * 3 * nn;
    const double* gb = gamma + (size_t)b * len;
    double* lam = lambda + (size_t)b * len;
    double* rv = (double*)malloc(len * sizeof(double));
    double* zv = (double*)malloc(len * sizeof(double));
    double* pv = (double*)malloc(len * sizeof(double));
    double* vv = (double*)malloc(len * sizeof(double));
    int fl = 0, it = 0;

    double gnorm = sqrt(dot(len, gb, gb));
    if (!isfinite(gnorm)) {
        fl |= REF_F_NONFINITE;
        iters[b] = 0;
        relres[b] = NAN;
        flags[b] |= fl;
        free(rv); free(zv); free(pv); free(vv);
        return;
    }
    if (gnorm == 0.0) {
        for (size_t i = 0; i < len; ++i) lam[i] = 0.0;
        iters[b] = 0;
        relres[b] = 0.0;
        free(rv); free(zv); free(pv); free(vv);
        return;
    }
    btd_mv(n, N, Sb, lam, vv);
    for (size_t i = 0; i < len; ++i) rv[i] = gb[i] - vv[i];
    double rr = dot(len, rv, rv);
    int converged = sqrt(rr) <= eps * gnorm;
    if (!isfinite(rr)) fl |= REF_F_NONFINITE;
    double eta = 0.0;
    if (!converged && !(fl & REF_F_NONFINITE)) {
        btd_mv(n, N, Pb, rv, zv);
        for (size_t i = 0; i < len; ++i) pv[i] = zv[i];
        eta = dot(len, rv, zv);
        while (it < max_iters) {
            btd_mv(n, N, Sb, pv, vv);
            double pSp = dot(len, pv, vv);
            if (!isfinite(pSp)) { fl |= REF_F_NONFINITE; break; }
            if (!(pSp > 0.0)) { fl |= REF_F_PCG_BREAKDOWN; break; }
            double a = eta / pSp;
            for (size_t i = 0; i < len; ++i) {
                lam[i] += a * pv[i];
                rv[i] -= a * vv[i];
            }
            ++it;
            rr = dot(len, rv, rv);
            if (!isfinite(rr)) { fl |= REF_F_NONFINITE; break; }
            if (sqrt(rr) <= eps * gnorm) { converged = 1; break; }
            btd_mv(n, N, Pb, rv, zv);
            double eta1 = dot(len, rv, zv);
            if (!isfinite(eta1)) { fl |= REF_F_NONFINITE; break; }
            double beta = eta1 / eta;
            for (size_t i = 0; i < len; ++i) pv[i] = zv[i] + beta * pv[i];
            eta = eta1;
        }
        if (!converged && !(fl & (REF_F_NONFINITE | REF_F_PCG_BREAKDOWN)))
            fl |= REF_F_PCG_MAXITER;
    }
    iters[b] = it;
    relres[b] = sqrt(rr) / gnorm;
    flags[b] |= fl;
    free(rv); free(zv); free(pv); free(vv);
}

/*
 * Recovery of the primal step from the multipliers, dz = G^-1 (C' lambda - g)
 * (the back-substitution half of the Schur solve, eq. 4):
 *   dx_k = Q~_k^-1 (lambda_k - A_k' lambda_{k+1} - q_k)      (k < N-1)
 *   dx_{N-1} = Q~_{N-1}^-1 (lambda_{N-1} - q_{N-1})
 *   du_k = R_k^-1 (-B_k' lambda_{k+1} - r_k).
 */
static void recover_one(const gato_ref_dims* d, int b, const double* Qinv, const double* Rinv,
                        const double* A, const double* Bu, const double* q, const double* r,
                        const double* lambda, double* dz)
{
    const int n = d->n, m = d->m, N = d->N;
    const size_t nn = (size_t)n * n, mm_ = (size_t)m * m, nm = (size_t)n * m;
    const size_t nz = (size_t)N * n + (size_t)(N - 1) * m;
    const double* lam = lambda + (size_t)b * N * n;
    double* dzb = dz + (size_t)b * nz;
    double* w = (double*)malloc((size_t)(n > m ? n : m) * sizeof(double));
    double* t = (double*)malloc((size_t)(n > m ? n : m) * sizeof(double));
    for (int k = 0; k < N; ++k) {
        double* dx = dzb + (size_t)k * (n + m);
        for (int i = 0; i < n; ++i) w[i] = lam[(size_t)k * n + i] - q[((size_t)b * N + k) * n + i];
        if (k < N - 1) {
            mtv(n, n, A + ((size_t)b * (N - 1) + k) * nn, lam + (size_t)(k + 1) * n, t);
            for (int i = 0; i < n; ++i) w[i] -= t[i];
        }
        mv(n, n, Qinv + ((size_t)b * N + k) * nn, w, dx);
        if (k < N - 1) {
            double* du = dx + n;
            mtv(n, m, Bu + ((size_t)b * (N - 1) + k) * nm, lam + (size_t)(k + 1) * n, t);
            for (int i = 0; i < m; ++i) w[i] = -t[i] - r[((size_t)b * (N - 1) + k) * m + i];
            mv(m, m, Rinv + ((size_t)b * (N - 1) + k) * mm_, w, du);
        }
    }
    free(w);
    free(t);
}

int gato_ref_pcg_solve(const gato_ref_dims* d, const double* S, const double* Pinv,
                       const double* gamma, const double* Qinv, const double* Rinv,
                       const double* A, const double* Bu, const double* q, const double* r,
                       double eps, int max_iters, double* lambda, double* dz, int* iters,
                       double* relres, int* flags)
{
    if (!d || d->n < 1 || d->m < 1 || d->N < 1 || d->B < 0) return -2;
    if (!(eps > 0.0) || max_iters < 1) return -4;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < d->B; ++b) {
        pcg_one(d, b, S, Pinv, gamma, eps, max_iters, lambda, iters, relres, flags);
        recover_one(d, b, Qinv, Rinv, A, Bu, q, r, lambda, dz);
    }
    return 0;
}

/*
 * Exact multipliers by a block Cholesky (block Thomas) factorisation of the
 * block-tridiagonal S -- the chronological elimination the Branch page
 * describes for time-ordered frames -- used to check PCG's answer, not by
 * the method itself.  S = L L' with L block lower bidiagonal:
 *   L_00 L_00' = D_0;  L_{k+1,k} = S_{k+1,k} L_kk^-T;
 *   L_{k+1,k+1} L_{k+1,k+1}' = D_{k+1} - L_{k+1,k} L_{k+1,k}'.
 * Returns the S_NOT_SPD flag bit when a pivot is not positive.
 */
static int chol_lower(int p, double* M) /* in place, lower factor; upper part zeroed */
{
    int bad = 0;
    for (int j = 0; j < p; ++j) {
        double dd = M[j * p + j];
        for (int l = 0; l < j; ++l) dd -= M[j * p + l] * M[j * p + l];
        if (!(dd > 0.0) || !isfinite(dd)) bad = 1;
        double ljj = sqrt(dd);
        M[j * p + j] = ljj;
        for (int i = j + 1; i < p; ++i) {
            double s = M[i * p + j];
            for (int l = 0; l < j; ++l) s -= M[i * p + l] * M[j * p + l];
            M[i * p + j] = s / ljj;
        }
        for (int i = 0; i < j; ++i) M[i * p + j] = 0.0;
    }
    return bad;
}

static void direct_one(const gato_ref_dims* d, int b, const double* S, const double* gamma,
                       double* lambda, int* flags)
{
    const int n = d->n, N = d->N;
    const size_t nn = (size_t)n * n;
    const double* Sb = S + (size_t)b * N * 3 * nn;
    const double* gb = gamma + (size_t)b * N * n;
    double* lam = lambda + (size_t)b * N * n;
    double* Ld = (double*)malloc((size_t)N * nn * sizeof(double)); /* L_kk */
    double* Lo = (double*)calloc((size_t)N * nn, sizeof(double));  /* L_{k,k-1} */
    double* y = (double*)malloc((size_t)N * n * sizeof(double));
    int fl = 0;
    for (int k = 0; k < N; ++k) {
        double* Lkk = Ld + k * nn;
        for (size_t i = 0; i < nn; ++i) Lkk[i] = Sb[((size_t)k * 3 + 1) * nn + i];
        if (k > 0) {
            /* L_{k,k-1} = S_{k,k-1} L_{k-1,k-1}^-T: row i solves L_{k-1,k-1} x = S row i. */
            const double* Lp = Ld + (size_t)(k - 1) * nn;
            double* Lok = Lo + k * nn;
            const double* Slo = Sb + ((size_t)k * 3 + 0) * nn;
            for (int i = 0; i < n; ++i)
                for (int j = 0; j < n; ++j) {
                    double s = Slo[i * n + j];
                    for (int l = 0; l < j; ++l) s -= Lok[i * n + l] * Lp[j * n + l];
                    Lok[i * n + j] = s / Lp[j * n + j];
                }
            for (int i = 0; i < n; ++i)
                for (int j = 0; j < n; ++j) {
                    double s = 0.0;
                    for (int l = 0; l < n; ++l) s += Lok[i * n + l] * Lok[j * n + l];
                    Lkk[i * n + j] -= s;
                }
        }
        if (chol_lower(n, Lkk)) fl |= REF_F_S_NOT_SPD;
    }
    /* Forward: L y = gamma. */
    for (int k = 0; k < N; ++k)
        for (int i = 0; i < n; ++i) {
            double s = gb[(size_t)k * n + i];
            if (k > 0)
                for (int l = 0; l < n; ++l) s -= Lo[k * nn + i * n + l] * y[(size_t)(k - 1) * n + l];
            for (int l = 0; l < i; ++l) s -= Ld[k * nn + i * n + l] * y[(size_t)k * n + l];
            y[(size_t)k * n + i] = s / Ld[k * nn + i * n + i];
        }
    /* Backward: L' lambda = y. */
    for (int k = N - 1; k >= 0; --k)
        for (int i = n - 1; i >= 0; --i) {
            double s = y[(size_t)k * n + i];
            if (k < N - 1)
                for (int l = 0; l < n; ++l)
                    s -= Lo[(size_t)(k + 1) * nn + l * n + i] * lam[(size_t)(k + 1) * n + l];
            for (int l = i + 1; l < n; ++l) s -= Ld[k * nn + l * n + i] * lam[(size_t)k * n + l];
            lam[(size_t)k * n + i] = s / Ld[k * nn + i * n + i];
        }
    flags[b] |= fl;
    free(Ld); free(Lo); free(y);
}

int gato_ref_direct_solve(const gato_ref_dims* d, const double* S, const double* gamma,
                          double* lambda, int* flags)
{
    if (!d || d->n < 1 || d->N < 1 || d->B < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < d->B; ++b) direct_one(d, b, S, gamma, lambda, flags);
    return 0;
}

/* Recovery alone (for checking the direct solve's dz against PCG's). */
int gato_ref_recover(const gato_ref_dims* d, const double* Qinv, const double* Rinv,
                     const double* A, const double* Bu, const double* q, const double* r,
                     const double* lambda, double* dz)
{
    if (!d || d->n < 1 || d->m < 1 || d->N < 1 || d->B < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < d->B; ++b) recover_one(d, b, Qinv, Rinv, A, Bu, q, r, lambda, dz);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Stage 3: L1 merit at the line-search step sizes (Sec. II eq. 3,     */
/* Sec. III eq. 7) and the selection                                  */
/* ------------------------------------------------------------------ */

/*
 * Merit of the trial point Z + alpha dZ, evaluated directly from its
 * definition (reading of eq. 3): the quadratic cost model of the step
 * (undamped Q: rho only regularises the step computation) plus mu times the
 * L1 norm of the linearised constraint violation at the trial point,
 *   M(alpha) = sum_k [ q_k'(a dx_k) + 1/2 (a dx_k)'Q_k(a dx_k) ]
 *            + sum_{k<N-1} [ r_k'(a du_k) + 1/2 (a du_k)'R_k(a du_k) ]
 *            + mu ( ||x0 - a dx_0||_1
 *                 + sum_{k<N-1} ||e_k + A_k(a dx_k) + B_k(a du_k) - a dx_{k+1}||_1 ).
 * The cost's value at the nominal point is taken as zero (the synthetic
 * problem is the LQ model itself).  M(0) = mu ||c||_1 is reported as merit0.
 * Selection (reading of eq. 7 with the GATO docs' failed line search): the
 * candidate of least merit, ties to the earlier (larger) step; accepted only
 * if it is below merit0, else best = -1 and the line-search-failed flag.
 */
static double merit_at(const gato_ref_dims* d, int b, const double* Q, const double* q,
                       const double* R, const double* r, const double* A, const double* Bu,
                       const double* e, const double* x0, const double* dz, double alpha,
                       double mu, double* xs, double* us, double* t)
{
    const int n = d->n, m = d->m, N = d->N;
    const size_t nn = (size_t)n * n, mm_ = (size_t)m * m, nm = (size_t)n * m;
    const size_t nz = (size_t)N * n + (size_t)(N - 1) * m;
    const double* dzb = dz + (size_t)b * nz;
    double cost = 0.0, viol = 0.0;
    for (int k = 0; k < N; ++k) {
        for (int i = 0; i < n; ++i) xs[i] = alpha * dzb[(size_t)k * (n + m) + i];
        const double* Qk = Q + ((size_t)b * N + k) * nn;
        const double* qk = q + ((size_t)b * N + k) * n;
        mv(n, n, Qk, xs, t);
        cost += dot((size_t)n, qk, xs) + 0.5 * dot((size_t)n, xs, t);
        if (k == 0)
            for (int i = 0; i < n; ++i) viol += fabs(x0[(size_t)b * n + i] - xs[i]);
        if (k < N - 1) {
            for (int i = 0; i < m; ++i) us[i] = alpha * dzb[(size_t)k * (n + m) + n + i];
            const double* Rk = R + ((size_t)b * (N - 1) + k) * mm_;
            const double* rk = r + ((size_t)b * (N - 1) + k) * m;
            mv(m, m, Rk, us, t);
            cost += dot((size_t)m, rk, us) + 0.5 * dot((size_t)m, us, t);
            const double* Ak = A + ((size_t)b * (N - 1) + k) * nn;
            const double* Bk = Bu + ((size_t)b * (N - 1) + k) * nm;
            const double* ek = e + ((size_t)b * (N - 1) + k) * n;
            const double* dxn = dzb + (size_t)(k + 1) * (n + m);
            for (int i = 0; i < n; ++i) {
                double s = ek[i] - alpha * dxn[i];
                for (int l = 0; l < n; ++l) s += Ak[i * n + l] * xs[l];
                for (int l = 0; l < m; ++l) s += Bk[i * m + l] * us[l];
                viol += fabs(s);
            }
        }
    }
    return cost + mu * viol;
}

int gato_ref_merit_eval(const gato_ref_dims* d, const double* Q, const double* q, const double* R,
                        const double* r, const double* A, const double* Bu, const double* e,
                        const double* x0, const double* dz, const double* alphas, int n_alpha,
                        double mu, double* merit, double* merit0, int* best, int* flags)
{
    if (!d || d->n < 1 || d->m < 1 || d->N < 1 || d->B < 0) return -2;
    if (n_alpha < 1 || !(mu >= 0.0)) return -4;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < d->B; ++b) {
        const int p = d->n > d->m ? d->n : d->m;
        double* xs = (double*)malloc((size_t)d->n * sizeof(double));
        double* us = (double*)malloc((size_t)(d->m > 0 ? d->m : 1) * sizeof(double));
        double* t = (double*)malloc((size_t)p * sizeof(double));
        double m0 = merit_at(d, b, Q, q, R, r, A, Bu, e, x0, dz, 0.0, mu, xs, us, t);
        merit0[b] = m0;
        int bi = 0;
        double bv = 0.0;
        for (int i = 0; i < n_alpha; ++i) {
            double v = merit_at(d, b, Q, q, R, r, A, Bu, e, x0, dz, alphas[i], mu, xs, us, t);
            merit[(size_t)b * n_alpha + i] = v;
            if (i == 0 || v < bv) { bv = v; bi = i; }
        }
        if (bv < m0) {
            best[b] = bi;
        } else {
            best[b] = -1;
            flags[b] |= REF_F_LS_FAILED;
        }
        free(xs); free(us); free(t);
    }
    return 0;
}

/* One SQP iteration's linear-algebra core: form -> PCG -> recover -> merit. */
int gato_ref_sqp_step(const gato_ref_dims* d, const double* Q, const double* q, const double* R,
                      const double* r, const double* A, const double* Bu, const double* e,
                      const double* x0, const double* rho, double eps, int max_iters,
                      const double* alphas, int n_alpha, double mu, double* lambda, double* dz,
                      double* merit, double* merit0, int* best, int* iters, double* relres,
                      int* flags)
{
    if (!d || d->n < 1 || d->m < 1 || d->N < 1 || d->B < 0) return -2;
    if (!(eps > 0.0) || max_iters < 1 || n_alpha < 1 || !(mu >= 0.0)) return -4;
    const size_t nn = (size_t)d->n * d->n, mm_ = (size_t)d->m * d->m;
    const size_t B = (size_t)d->B, N = (size_t)d->N;
    double* S = (double*)malloc(B * N * 3 * nn * sizeof(double) + 1);
    double* P = (double*)malloc(B * N * 3 * nn * sizeof(double) + 1);
    double* g = (double*)malloc(B * N * d->n * sizeof(double) + 1);
    double* Qi = (double*)malloc(B * N * nn * sizeof(double) + 1);
    double* Ri = (double*)malloc(B * (N - 1) * mm_ * sizeof(double) + 1);
    int rc = gato_ref_form_schur(d, Q, q, R, r, A, Bu, e, x0, rho, S, P, g, Qi, Ri, flags);
    if (rc == 0)
        rc = gato_ref_pcg_solve(d, S, P, g, Qi, Ri, A, Bu, q, r, eps, max_iters, lambda, dz, iters,
                                relres, flags);
    if (rc == 0)
        rc = gato_ref_merit_eval(d, Q, q, R, r, A, Bu, e, x0, dz, alphas, n_alpha, mu, merit,
                                 merit0, best, flags);
    free(S); free(P); free(g); free(Qi); free(Ri);
    return rc;
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of host threads the OpenMP loops over solves will use. */
int gato_ref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set that number (for timing the oracle on fewer cores); returns the new value.
 * Scheduling only: every solve is computed by one thread, whichever. */
int gato_ref_set_num_threads(int t)
{
#ifdef _OPENMP
    if (t >= 1) omp_set_num_threads(t);
    return omp_get_max_threads();
#else
    (void)t;
    return 1;
#endif
}
