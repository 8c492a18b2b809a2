/*
 * gato_driver.h -- device-side pieces of the multi-iteration SQP driver around
 * gato_sqp_step (the outer loop of the GATO paper, Sec. III-IV: per iteration,
 * linearise about the current trajectory, one SQP step, take the selected step,
 * update the damping rho from the line search), so that an iteration is three
 * kernel launches: gato_chain_qp, gato_sqp_step, gato_take_step.
 *
 * Layouts, ownership, streams and errors are those of gato.h: fp32 device
 * arrays, batch-major, contiguous; every call only enqueues work on `stream`;
 * host-side validation returns a negative GATO_E_* code before anything is
 * enqueued (NULL pointer, bad dims or parameters); B = 0 returns GATO_OK.
 *   X [B][N][n]   U [B][N-1][m]   x_init, x_ref [B][n]   rho [B]
 */
#ifndef GATO_DRIVER_H
#define GATO_DRIVER_H

#include "gato.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The analytic plant the driver runs on (a synthetic stand-in for the robot
 * models the GATO pages linearise with GRiD): a chain of d coupled, damped
 * pendulums, state x = [theta (d), omega (d)], control u (d torques), so
 * n = 2d and m = d, stepped by explicit Euler with step h:
 *   theta' = theta + h omega,
 *   omega' = omega + h (-a sin(theta) - c omega + kappa L theta + u),
 * with L the path-graph Laplacian over the joints (free ends: -1 at both ends
 * of its diagonal, -2 inside, 1 beside it).  Cost per knot:
 *   1/2 (x - x_ref)' diag(w_theta I, w_omega I) (x - x_ref) + 1/2 w_u u'u. */
typedef struct {
    int32_t dof;
    float h, a, c, kappa, w_theta, w_omega, w_u;
} gato_chain_t;

/* The QP of one SQP iteration at the trajectory (X, U) (GATO paper Sec. II,
 * Step 1), for every solve and knot:
 *   A_k = df/dx (x_k, u_k) = [[I, h I], [h (-a diag(cos theta_k) + kappa L), (1 - h c) I]],
 *   B_k = df/du = [[0], [h I]],   e_k = f(x_k, u_k) - x_{k+1}   (k < N-1),
 *   Q_k = diag(w_theta I, w_omega I),  q_k = Q_k (x_k - x_ref),
 *   R_k = w_u I,  r_k = w_u u_k,  x0 = x_init - x_0,
 * written in gato_sqp_step's input layouts (dims->n must be 2 dof and
 * dims->m must be dof, else GATO_E_DIMS). */
int gato_chain_qp(const gato_dims_t* dims, const gato_chain_t* plant, const float* X, const float* U,
                  const float* x_init, const float* x_ref, float* Q, float* q, float* R, float* r, float* A,
                  float* Bu, float* e, float* x0, hipStream_t stream);

/* The selected step and the damping update after gato_sqp_step:
 *   a = alphas[best] (0 when best < 0, a failed line search),
 *   X += a dX,  U += a dU   (dz = [dx_0 du_0 ... dx_{N-1}], gato.h's layout),
 *   rho = max(rho / 10, rho_min) after a full step (best = 0),
 *         min(rho * 10, rho_max) after a failed line search, unchanged otherwise
 * (the driver's damping schedule; the pages tie rho to the line search's
 * outcome without printing the rule).  alphas_host: the step sizes of the
 * step call (at most GATO_MAX_ALPHA), copied by value; a best beyond them is
 * taken as a failed line search. */
int gato_take_step(const gato_dims_t* dims, const float* alphas_host, int32_t n_alpha, const float* dz,
                   const int32_t* best, float* X, float* U, float* rho, float rho_min, float rho_max,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GATO_DRIVER_H */
