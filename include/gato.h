/*
 * gato.h -- C ABI of libgato.so: one SQP iteration's linear-algebra core over
 * a batch of independent LQ subproblems, on one AMD Instinct MI355X (gfx950).
 *
 * The method is the one "GATO: GPU-Accelerated and Batched Trajectory
 * Optimization for Scalable Edge Model Predictive Control" (arXiv 2510.07625)
 * describes in Sec. II-III:
 *   (1) form the block-tridiagonal Schur complement S, the vector gamma and the
 *       symmetric stair preconditioner Phi^-1 from the QP data (eqs. 4-6);
 *   (2) solve S lambda = gamma by preconditioned conjugate gradient, one solve
 *       per workgroup, and recover the primal step dz;
 *   (3) evaluate the L1 merit function at the line-search step sizes for every
 *       knot and solve and reduce them (eqs. 3 and 7).
 *
 * ---------------------------------------------------------------- problem
 * Per solve b (B solves, N knot points, n states, m controls), the QP is
 *   min  sum_{k<N} 1/2 dx_k'(Q_k + rho_b I)dx_k + q_k'dx_k
 *      + sum_{k<N-1} 1/2 du_k'R_k du_k + r_k'du_k
 *   s.t. dx_0 = x0,  dx_{k+1} = A_k dx_k + B_k du_k + e_k   (k < N-1),
 * with e_k = f(x_k,u_k,h) - x_{k+1} the dynamics defect (GATO paper Sec. II,
 * Step 1).  The pages number states x_0..x_N; here N counts knot points, so
 * states are x_0..x_{N-1} and controls u_0..u_{N-2}.
 *
 * ---------------------------------------------------------------- layouts
 * Every array is fp32, row-major, batch-major, contiguous and unpadded
 * (the dense contiguous packing by batch and knot of the paper's Sec. III):
 *   Q    [B][N][n][n]      q   [B][N][n]
 *   R    [B][N-1][m][m]    r   [B][N-1][m]
 *   A    [B][N-1][n][n]    Bu  [B][N-1][n][m]    e [B][N-1][n]    x0 [B][n]
 *   rho  [B]  (nullable: no damping)
 *   S, Pinv [B][N][3][n][n]  block row k = [X_{k,k-1}, X_{k,k}, X_{k,k+1}];
 *                            out-of-range blocks (k = 0 left, k = N-1 right)
 *                            are written as zeros
 *   gamma, lambda [B][N][n]   Qinv [B][N][n][n]   Rinv [B][N-1][m][m]
 *   dz   [B][N*n + (N-1)*m]  ordered dx_0, du_0, dx_1, du_1, ..., dx_{N-1}
 *                            (dz_k = [dx_k du_k], the paper's Step 2 ordering)
 *   merit [B][n_alpha]   merit0 [B]   best [B] (int32)
 *   iters [B] (int32)    relres [B]   flags [B] (int32, GATO_F_* bits)
 *
 * ---------------------------------------------------------------- ownership
 * All array arguments except alphas_host are device pointers owned by the
 * caller (e.g. from torch tensors); the library never allocates, frees or
 * copies host<->device inside a call.  alphas_host is a host array of at most
 * GATO_MAX_ALPHA floats, copied by value into the launch.  Outputs must not
 * alias inputs, except lambda, which is read (warm start) and written.
 *
 * ---------------------------------------------------------------- streams
 * Every call only enqueues work on `stream` and returns; outputs are valid
 * after the stream is synchronised.  Exception: gato_sqp_step with a non-NULL
 * `times` records events and synchronises the stream before returning.
 *
 * ---------------------------------------------------------------- errors
 * Host-side validation runs before anything is enqueued and returns a
 * negative GATO_E_* code (nothing enqueued) for: a NULL required pointer,
 * dims < 1, a shape (n, m, N) the call does not serve (GATO_E_UNSUPPORTED;
 * see gato_shape_supported), a pointer not 4-byte aligned,
 * eps <= 0, max_iters < 1, n_alpha outside [1, GATO_MAX_ALPHA], mu < 0 or a
 * workspace smaller than gato_workspace_bytes().  B = 0 returns GATO_OK
 * once the dims are valid, before any pointer is looked at (empty tensors may
 * have NULL data).  With N = 1 the arrays indexed by the dynamics (R, r, A,
 * Bu, e, Rinv) are empty and may be NULL.  A failed launch returns
 * GATO_E_HIP.  Numerical trouble never makes a call fail: it sets per-solve
 * flag bits and the solve's outputs are still written (a failed pivot is
 * flagged, not repaired).  gato_form_schur and gato_sqp_step set flags[b];
 * gato_pcg_solve and gato_merit_eval OR their bits into it.
 *
 * The library keeps no global mutable state: calls on different streams or
 * threads are independent.
 */
#ifndef GATO_H
#define GATO_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GATO_MAX_ALPHA 16

typedef struct {
    int32_t n; /* states per knot */
    int32_t m; /* controls per knot */
    int32_t N; /* knot points (horizon) */
    int32_t B; /* independent solves in the batch */
} gato_dims_t;

/* Device time per stage of gato_sqp_step, in microseconds (the stage split
 * of the GATO docs' solver statistics: schur / linsys / merit). */
typedef struct {
    float schur_us;
    float linsys_us;
    float merit_us;
    float total_us;
} gato_stage_times_t;

enum {
    GATO_OK = 0,
    GATO_E_NULL = -1,
    GATO_E_DIMS = -2,
    GATO_E_ALIGN = -3,
    GATO_E_PARAM = -4,
    GATO_E_HIP = -5,
    GATO_E_UNSUPPORTED = -6,
    GATO_E_WORKSPACE = -7
};

enum {
    GATO_F_Q_NOT_SPD = 1,       /* a pivot of Q_k + rho I was not positive */
    GATO_F_R_NOT_SPD = 2,       /* a pivot of R_k was not positive */
    GATO_F_S_NOT_SPD = 4,       /* a pivot of a diagonal Schur block D_k was not positive */
    GATO_F_PCG_MAXITER = 8,     /* PCG stopped at max_iters without meeting eps */
    GATO_F_PCG_BREAKDOWN = 16,  /* p'S p <= 0 in PCG */
    GATO_F_LS_FAILED = 32,      /* no step size lowered the merit below merit0 */
    GATO_F_NONFINITE = 64       /* a PCG reduction was not finite */
};

/*
 * Stage 1 (GATO paper Sec. II eqs. 4-6; setup kernel of Sec. III).
 * With Q~_k = Q_k + rho_b I:
 *   Qinv_k = Q~_k^-1, Rinv_k = R_k^-1;
 *   D_0 = Q~_0^-1,  D_{k+1} = A_k Q~_k^-1 A_k' + B_k R_k^-1 B_k' + Q~_{k+1}^-1;
 *   S_{k,k+1} = -Q~_k^-1 A_k' = S_{k+1,k}';
 *   gamma_0 = x0 + Q~_0^-1 q_0,
 *   gamma_{k+1} = e_k - A_k Q~_k^-1 q_k - B_k R_k^-1 r_k + Q~_{k+1}^-1 q_{k+1};
 *   Phi^-1_{k,k} = D_k^-1,  Phi^-1_{k,k+1} = -D_k^-1 S_{k,k+1} D_{k+1}^-1 = Phi^-1_{k+1,k}'.
 * Writes S, Pinv, gamma, Qinv, Rinv and flags (Q/R/S_NOT_SPD bits).
 */
int gato_form_schur(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                    const float* r, const float* A, const float* Bu, const float* e,
                    const float* x0, const float* rho, float* S, float* Pinv, float* gamma,
                    float* Qinv, float* Rinv, int32_t* flags, hipStream_t stream);

/*
 * Stage 2 (GATO paper Sec. II, PCG on S lambda = gamma; batched solver of
 * Sec. III, one workgroup per solve).  From lambda (in) as the starting point:
 *   r = gamma - S lambda; z = Phi^-1 r; p = z; eta = r'z; then per iteration
 *   v = S p; a = eta / p'v; lambda += a p; r -= a v;
 *   stop when ||r||_2 <= eps ||gamma||_2;  z = Phi^-1 r; p = z + (r'z / eta) p.
 * ||gamma|| = 0 gives lambda = 0 after 0 iterations.  iters never exceeds
 * max_iters.  Within the horizon one workgroup holds, the assembled Phi^-1
 * blocks are applied; their fp32 values can be indefinite where cond(Phi^-1)
 * passes ~1e8, which shows as r'z <= 0 while the residual is above the
 * tolerance.  Such a solve switches at that iteration to Phi^-1 in the factored
 * form below and restarts from its current lambda with the iterations left of
 * max_iters (iters counts both runs).  Beyond the horizon one workgroup holds
 * (N > 64 for n <= 16, N > 16 for n <= 32) z = Phi^-1 r is always applied in the
 * preconditioner's factored form D^-1 (J S J) (D^-1 r), with D^-1 = the diagonal
 * blocks of Phi^-1 and J = blkdiag((-1)^k I): the same operator, which stays
 * positive definite in fp32 while S does even where the assembled fp32 Phi^-1
 * does not; it reads S and the diagonal blocks of Phi^-1.  Then the step
 *   dx_k = Qinv_k (lambda_k - A_k' lambda_{k+1} - q_k),  dx_{N-1} = Qinv_{N-1}(lambda_{N-1} - q_{N-1}),
 *   du_k = Rinv_k (-B_k' lambda_{k+1} - r_k),
 * evaluated as dx_k = Qinv_k lambda_k + S_{k,k+1} lambda_{k+1} - Qinv_k q_k, since
 * S_{k,k+1} = -Q~_k^-1 A_k'.  A is therefore not read and may be NULL (it is
 * kept in the argument list so that the call takes the QP data as the problem
 * states it); S, Qinv, q, Bu, Rinv and r must be those of one problem, as
 * gato_form_schur writes them.
 * Writes lambda, dz, iters (S-products in the loop), relres (recurred
 * ||r|| / ||gamma||) and ORs PCG_MAXITER / PCG_BREAKDOWN / NONFINITE into flags.
 */
int gato_pcg_solve(const gato_dims_t* dims, const float* S, const float* Pinv,
                   const float* gamma, const float* Qinv, const float* Rinv, const float* A,
                   const float* Bu, const float* q, const float* r, float eps, int32_t max_iters,
                   float* lambda, float* dz, int32_t* iters, float* relres, int32_t* flags,
                   hipStream_t stream);

/*
 * Stage 2, direct (the block-tridiagonal direct solve the GATO pages weigh
 * against PCG for long horizons; Branch's chronological elimination of a
 * block-structured KKT system).  Solves S lambda = gamma exactly (up to
 * rounding) by block elimination, the block LDL' factorisation of S:
 *   H_0 = D_0, g_0 = gamma_0;  T_k = S_{k,k-1} H_{k-1}^-1,
 *   H_k = D_k - T_k S_{k-1,k},  g_k = gamma_k - T_k g_{k-1};
 *   lambda_{N-1} = H_{N-1}^-1 g_{N-1},  lambda_k = H_k^-1 (g_k - S_{k,k+1} lambda_{k+1}),
 * then recovers dz exactly as gato_pcg_solve does.  Arguments as in
 * gato_pcg_solve, without a starting point, tolerance or iteration cap;
 * lambda and dz are outputs only.  H_k^-1 (Gauss-Jordan, no pivoting: every H_k
 * of an SPD S is SPD) and g_k are kept in the caller's workspace, of at least
 * gato_direct_workspace_bytes(dims) bytes, 256-byte aligned.  A pivot that is not
 * positive ORs S_NOT_SPD into flags, a non-finite lambda NONFINITE.  The knots are
 * walked in order, so a solve's time grows linearly with N and does not depend
 * on the conditioning of S.
 */
size_t gato_direct_workspace_bytes(const gato_dims_t* dims);
int gato_direct_solve(const gato_dims_t* dims, const float* S, const float* gamma, const float* Qinv,
                      const float* Rinv, const float* Bu, const float* q, const float* r, float* lambda,
                      float* dz, int32_t* flags, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Stage 2, cyclic reduction (the cyclic-frames elimination plan of the Branch
 * page, "Specializing Robotics Solvers in Warp": its elimination-plan figure
 * and the cyclic-reduction row of its plans table; the log-depth alternative
 * to gato_direct_solve for long horizons).  Solves S lambda = gamma exactly (up
 * to rounding) by block cyclic reduction: level l = 0, 1, ... eliminates the
 * knots that are odd multiples of s = 2^l from the system on the multiples of
 * s.  With L_k, U_k the couplings of knot k to knots k - s and k + s there,
 * an eliminated knot j forms Y1_j = D_j^-1 L_j, Y2_j = D_j^-1 U_j,
 * y3_j = D_j^-1 gamma_j, and a kept knot i (a multiple of 2s) becomes
 *   D_i - L_i Y2_{i-s} - U_i Y1_{i+s},  L_i <- -L_i Y1_{i-s},  U_i <- -U_i Y2_{i+s},
 *   gamma_i - L_i y3_{i-s} - U_i y3_{i+s}.
 * Knot 0 is left alone after ceil(log2 N) levels and solved directly; the
 * back substitution lambda_j = y3_j - Y1_j lambda_{j-s} - Y2_j lambda_{j+s}
 * runs the levels in reverse.  Then dz is recovered exactly as gato_pcg_solve
 * does.  Each elimination is a Cholesky factorisation of the pivot block with
 * a lower solve of its couplings, D_j = C C', W = C^-1 [L U gamma], followed by
 * the Schur update of the neighbours (the block Cholesky factorisation of S
 * with its knots reordered), so every pivot block is SPD when S is; a pivot
 * that is not positive ORs S_NOT_SPD into flags, a non-finite lambda NONFINITE.
 * For n <= 16 and N > 128 the order is a nested dissection: the horizon is cut
 * into 64 chunks whose interior knots are eliminated first, in order (each
 * chunk in parallel), and the 128 chunk-boundary knots are then reduced
 * cyclically as above.  For n <= 16 only the diagonal and upper blocks of S
 * are read (S is symmetric: S_{k,k-1} = S_{k-1,k}'); for n > 16 the lower
 * blocks too.  Arguments as in gato_direct_solve; the reduced rows
 * and factors go through the caller's workspace, of at least
 * gato_cr_workspace_bytes(dims) bytes, 256-byte aligned.  The eliminations of
 * one level (or chunk step) run in parallel, so a solve's depth grows with
 * log2 N (plus N/64 chunk steps) rather than N.
 */
size_t gato_cr_workspace_bytes(const gato_dims_t* dims);
int gato_cr_solve(const gato_dims_t* dims, const float* S, const float* gamma, const float* Qinv,
                  const float* Rinv, const float* Bu, const float* q, const float* r, float* lambda, float* dz,
                  int32_t* flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Number of levels of the cyclic-frames plan for a chain of N knots: ceil(log2 N)
 * reduction levels plus the final single-knot solve (0 for N < 1); gato_cr_solve
 * runs exactly these levels for N <= 128 (n <= 16) or any N (n > 16). */
int32_t gato_cr_levels(int32_t N);

/*
 * Stage 3 (GATO paper Sec. II eq. 3, Sec. III eq. 7; the merit kernel of the
 * GATO docs' "Merit launch timing").  For every solve, knot and step size a:
 *   m_k(a) = a (q_k'dx_k + r_k'du_k) + a^2/2 (dx_k'Q_k dx_k + du_k'R_k du_k)
 *          + mu ||e_k + a (A_k dx_k + B_k du_k - dx_{k+1})||_1   (k < N-1)
 *          + [k = 0] mu ||x0 - a dx_0||_1,
 * (undamped Q: rho regularises the step, not the merit), summed over knots in
 * a fixed pairwise order that does not depend on the launch shape, so results
 * are bit-identical for any workgroup size.  merit0 = M(0) = mu ||c||_1.
 * best = argmin_i merit[i] (ties to the smaller i) if below merit0, else -1
 * and LS_FAILED is ORed into flags.
 */
int gato_merit_eval(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                    const float* r, const float* A, const float* Bu, const float* e,
                    const float* x0, const float* dz, const float* alphas_host, int32_t n_alpha,
                    float mu, float* merit, float* merit0, int32_t* best, int32_t* flags,
                    hipStream_t stream);

/* Launch shapes of the merit (the GATO docs' "Merit launch timing": one block
 * per solve evaluating every candidate per knot, against one block per
 * candidate, at several block sizes).  gato_merit_eval with an explicit shape:
 *   variant GATO_MERIT_PER_KNOT: one workgroup per solve; each knot's
 *           step-size-independent products are formed once and every step size
 *           rescales them (gato_merit_eval's choice);
 *   variant GATO_MERIT_PER_CANDIDATE: one workgroup per (solve, step size, and
 *           the step size 0 of merit0), each recomputing the knot's products,
 *           then a selection kernel;
 *   waves:  wavefronts of 64 lanes per workgroup, 1..16, or 0 for
 *           gato_merit_eval's choice (enough for every knot at once, at most 16).
 * Every shape gives bit-identical merit, merit0, best and flags (the sums
 * over knots are the same canonical pairwise tree).  GATO_E_PARAM for an
 * unknown variant or waves outside [0, 16]. */
#define GATO_MERIT_PER_KNOT 0
#define GATO_MERIT_PER_CANDIDATE 1
int gato_merit_eval_shape(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                          const float* r, const float* A, const float* Bu, const float* e,
                          const float* x0, const float* dz, const float* alphas_host, int32_t n_alpha,
                          float mu, float* merit, float* merit0, int32_t* best, int32_t* flags,
                          int32_t variant, int32_t waves, hipStream_t stream);

/*
 * The three stages in one call (one SQP iteration's linear-algebra core,
 * GATO paper Sec. III, Fig. 2 steps a-c).  Outputs are those of the three
 * calls above; flags[b] is set (not ORed).  Horizon policy (the GATO pages'
 * choice between PCG and a block-tridiagonal direct solve by horizon, with the
 * switch point measured on this device):
 *  - where one workgroup can hold a whole solve (N <= 64 for n <= 16, N <= 16
 *    for n <= 32), the stages run fused in one kernel with PCG, and no
 *    workspace is used;
 *  - otherwise stage 2 is a direct solve: gato_cr_solve's block cyclic
 *    reduction while the batch is small enough for its log-depth to pay, else
 *    gato_direct_solve's block Thomas elimination (measured switch points: for
 *    n <= 16 and N <= 128, where the reduction refines on its own factors, the
 *    refined steps B * (0.220 + 0.00363 N) us < 3.6 N + 0.00465 N B us, or
 *    without the refinement pass the solves B * (0.15 + 0.00105 N) us <
 *    2.7 N us; B * (0.18 + 0.0019 N) us < 2.7 N us for n <= 16 beyond
 *    (B < ~1040-1300); B < ~400 for n > 16).  The direct solve is followed by one pass of
 *    iterative refinement of the KKT system (G dz - C' lambda = -g, C dz = c;
 *    the paper's eq. 2): its residual, accumulated in double from the problem
 *    data, is the right-hand side of a correction system with the same S,
 *    Q~^-1 and R^-1, whose gamma is formed from it and which the same
 *    factorisation of S solves; its lambda and dz are added to the first
 *    pass's.  The register-resident cyclic reduction (n <= 16, N <= 128) runs
 *    the pass inside its kernel on the factors of its first pass; the other
 *    direct solves run it as separate kernels and a second solve.  The fp32
 *    stages alone leave dz with a relative error of up to about
 *    cond(S) * 1e-7 (~1e-3 at cond(S) ~ 1e6, where rounding S to fp32 already
 *    moves dz by up to 6e-4); the pass brings it to ~1e-5.  The merit is
 *    evaluated on the refined dz; linsys_us includes the pass.
 *    lambda's input is not read, iters and relres are written as 0, and eps
 *    and max_iters are checked but unused.  S (no Phi^-1: the
 *    direct solves do not use it), gamma, Qinv, Rinv, the solve's rows, the
 *    refinement pass's buffers and the merit's per-knot values go through
 *    `workspace` (gato_workspace_bytes() bytes, 256-byte aligned,
 *    caller-owned device memory).  With a small batch the merit then spreads
 *    a solve's knots over several workgroups and sums their values in a
 *    second kernel, in the same canonical order (identical bits).
 * times (nullable): per-stage device times; when given, the call synchronises.
 */
int gato_sqp_step(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                  const float* r, const float* A, const float* Bu, const float* e,
                  const float* x0, const float* rho, float eps, int32_t max_iters,
                  const float* alphas_host, int32_t n_alpha, float mu, float* lambda, float* dz,
                  float* merit, float* merit0, int32_t* best, int32_t* iters, float* relres,
                  int32_t* flags, void* workspace, size_t workspace_bytes,
                  gato_stage_times_t* times, hipStream_t stream);

/* Stage-2 solvers of gato_sqp_step (gato_step_solver's result, and a choice
 * in gato_step_opts_t). */
#define GATO_SOLVER_AUTO (-1)     /* the horizon policy above */
#define GATO_SOLVER_FUSED_PCG 0   /* one fused kernel with PCG */
#define GATO_SOLVER_THOMAS 1      /* block Thomas (gato_direct_solve) */
#define GATO_SOLVER_CR 2          /* block cyclic reduction (gato_cr_solve) */
#define GATO_SOLVER_CR_STREAM 3   /* block cyclic reduction with every level's rows in the
                                     workspace (the kernel n > 16 always uses) */

/* Per-call choices of gato_sqp_step_opts.  They select among kernels and
 * passes; none of them changes the problem solved.
 *   solver: GATO_SOLVER_AUTO (the horizon policy), or a direct solve that
 *           then runs at every horizon, the fused ones included:
 *           GATO_SOLVER_THOMAS, GATO_SOLVER_CR or GATO_SOLVER_CR_STREAM.
 *           PCG stops at ||r|| <= eps ||gamma||, which bounds dz only to
 *           about cond(S) * eps; on ill-conditioned problems within the
 *           fused horizon (cond(S) ~ 1e6, N = 64) the PCG step lies within
 *           ~5e-4 of the exact step, a direct solve with its refinement pass
 *           within ~5e-6.  Such a call needs the workspace
 *           gato_step_workspace_bytes() gives.
 *   refine: 1 (the default of gato_sqp_step) runs the KKT refinement pass
 *           after a direct solve, 0 leaves the fp32 direct solve's step as
 *           it is; ignored on the fused path. */
typedef struct {
    int32_t solver;
    int32_t refine;
} gato_step_opts_t;

/* gato_sqp_step with explicit choices: arguments and outputs as there, plus
 * opts (nullable: {GATO_SOLVER_AUTO, 1}, i.e. exactly gato_sqp_step).  An
 * unknown solver or a refine outside {0, 1} returns GATO_E_PARAM. */
int gato_sqp_step_opts(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                       const float* r, const float* A, const float* Bu, const float* e,
                       const float* x0, const float* rho, float eps, int32_t max_iters,
                       const float* alphas_host, int32_t n_alpha, float mu, float* lambda, float* dz,
                       float* merit, float* merit0, int32_t* best, int32_t* iters, float* relres,
                       int32_t* flags, void* workspace, size_t workspace_bytes,
                       gato_stage_times_t* times, const gato_step_opts_t* opts, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gato_sqp_step without a workspace argument or stage times.  Where
 * gato_sqp_step needs a workspace (horizons beyond the fused ones), this call
 * uses a fixed array of GATO_NOALLOC_SCRATCH_BYTES in device memory that the
 * library holds on each GPU it runs on, from the first use there until the
 * process ends; it allocates nothing and calls no allocating routine.  Dims
 * whose gato_workspace_bytes() exceed that size return GATO_E_WORKSPACE
 * (before anything is enqueued).  The array of the calling thread's current
 * device is used, so `stream` must belong to that device.  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  Nothing in the
 * array needs to start at zero (every row is written before it is read), and
 * each call leaves its own values there.  Results are those of gato_sqp_step
 * (the same kernels in the same order).  A failed lookup of the array returns
 * GATO_E_HIP.
 */
#define GATO_NOALLOC_SCRATCH_BYTES (64u << 20)
int gato_sqp_step_noalloc(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                          const float* r, const float* A, const float* Bu, const float* e,
                          const float* x0, const float* rho, float eps, int32_t max_iters,
                          const float* alphas_host, int32_t n_alpha, float mu, float* lambda, float* dz,
                          float* merit, float* merit0, int32_t* best, int32_t* iters, float* relres,
                          int32_t* flags, hipStream_t stream);

/* The stage-2 solver gato_sqp_step runs for these dims (the horizon policy
 * above, a pure function of dims): GATO_SOLVER_FUSED_PCG, GATO_SOLVER_THOMAS or
 * GATO_SOLVER_CR; a negative status for invalid or unsupported dims. */
int gato_step_solver(const gato_dims_t* dims);

/* Workspace gato_sqp_step needs for these dims (0 when the fused path applies to
 * a shape with kernels of its own; the padded copies otherwise, see
 * gato_shape_supported). */
size_t gato_workspace_bytes(const gato_dims_t* dims, int32_t n_alpha);

/* The workspace gato_sqp_step_opts needs with these choices (opts nullable:
 * then, as with GATO_SOLVER_AUTO, gato_workspace_bytes()); a direct solver
 * within the fused horizon needs one where the fused path needs none.  0 for
 * invalid dims, B = 0, choices that need no workspace, or choices
 * gato_sqp_step_opts rejects (GATO_E_PARAM there). */
size_t gato_step_workspace_bytes(const gato_dims_t* dims, int32_t n_alpha, const gato_step_opts_t* opts);

/* Static description of a status code. */
const char* gato_status_string(int code);

/* Whether the library serves (n, m, N): 1 if it has kernels for (n, m), which are
 * (14,7), (12,6), (24,12), (4,2), (1,1) and (28,14), and 1 <= N <= 1024;
 * 2 if only the step calls (gato_sqp_step, gato_sqp_step_opts,
 * gato_sqp_step_noalloc) serve it, by padding; 0 otherwise.  Padding: a shape
 * without kernels, n <= 28 and m <= 14, is solved inside the smallest compiled
 * shape (n', m') with n' >= n and m' >= m (fewest states, then fewest controls):
 * Q_k and R_k get identity rows and columns beyond n and m, and A_k, B_k, q,
 * r, e, x0 and lambda's input zeros.  The added states and controls then form a
 * separate part of the QP whose solution is exactly zero, so the original
 * problem's dz, lambda, merits, selection, iterations and flags are the padded
 * problem's at the original rows.  The padded copies go through the step's
 * workspace (gato_workspace_bytes counts them, on the fused path too) and cost
 * two light copy kernels; stage times, when asked for, cover the padded step.
 * gato_pcg_solve alone is further limited to N <= 256 for n <= 16 and N <= 64
 * for n <= 32 (four knots per lane group) and returns GATO_E_UNSUPPORTED beyond;
 * the stage calls return GATO_E_UNSUPPORTED for shapes served by padding. */
int gato_shape_supported(int32_t n, int32_t m, int32_t N);

#ifdef __cplusplus
}
#endif

#endif /* GATO_H */
