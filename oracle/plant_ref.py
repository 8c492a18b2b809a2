"""fp64 reference of the SQP driver's analytic plant (test infrastructure only): the
chain of coupled, damped pendulums whose parameters block_tridiagonal_pcg_amd.synth.Chain
holds, written out in numpy.  Explicit Euler with step h:
    theta' = theta + h omega
    omega' = omega + h (-a sin(theta) - c omega + kappa L theta + u)
with L the path-graph Laplacian over the joints (free ends), and the tracking cost
1/2 (x - x_ref)' W (x - x_ref) + 1/2 u' Rw u with W = diag(w_theta I, w_omega I),
Rw = w_u I.  Arrays are batched: X [B][N][n], U [B][N-1][m].  Used by the reference
driver (driver_ref) to form each SQP iteration's QP data (the GATO paper's Sec. II,
Step 1: linearise about the current trajectory); its Jacobians are pinned against
central differences and its cost terms against the cost's gradient in the tests.
"""
import numpy as np


def laplacian_matrix(d):
    L = -2.0 * np.eye(d)
    for j in range(d - 1):
        L[j, j + 1] = L[j + 1, j] = 1.0
    L[0, 0] += 1.0
    L[d - 1, d - 1] += 1.0
    return L


def step(P, X, U):
    """f(x_k, u_k) for every knot that has a control: [B][N-1][n]."""
    d = P.dof
    th, om = X[..., :-1, :d], X[..., :-1, d:]
    acc = -P.a * np.sin(th) - P.c * om + P.kappa * (th @ laplacian_matrix(d)) + U
    return np.concatenate([th + P.h * om, om + P.h * acc], -1)


def linearize(P, X, U):
    """A_k = df/dx, B_k = df/du at (x_k, u_k), and the defects e_k = f(x_k, u_k) - x_{k+1}."""
    d, n = P.dof, P.n
    th = X[..., :-1, :d]
    shape = tuple(th.shape[:-1])
    eye = np.eye(d)
    A = np.zeros(shape + (n, n))
    Bu = np.zeros(shape + (n, d))
    A[..., :d, :d] = eye
    A[..., :d, d:] = P.h * eye
    A[..., d:, :d] = P.h * (-P.a * np.cos(th)[..., :, None] * eye + P.kappa * laplacian_matrix(d))
    A[..., d:, d:] = (1.0 - P.h * P.c) * eye
    Bu[..., d:, :] = P.h * eye
    e = step(P, X, U) - X[..., 1:, :]
    return A, Bu, e


def cost_terms(P, X, U, x_ref):
    """Q_k = W, q_k = W (x_k - x_ref), R_k = Rw, r_k = Rw u_k for the tracking cost."""
    d, n = P.dof, P.n
    w = np.concatenate([np.full(d, P.w_theta), np.full(d, P.w_omega)])
    Q = np.broadcast_to(np.diag(w), tuple(X.shape[:-1]) + (n, n)).copy()
    R = np.broadcast_to(P.w_u * np.eye(d), tuple(U.shape[:-1]) + (d, d)).copy()
    q = (X - x_ref[:, None, :]) * w
    r = P.w_u * U
    return Q, q, R, r


def defect(P, X, U, x_init):
    """Nonlinear constraint violation per solve: sum_k ||f(x_k,u_k) - x_{k+1}||_1 + ||x_init - x_0||_1."""
    e = step(P, X, U) - X[..., 1:, :]
    return np.abs(e).sum((-1, -2)) + np.abs(x_init - X[..., 0, :]).sum(-1)


def cost(P, X, U, x_ref):
    d = P.dof
    dx = X - x_ref[:, None, :]
    return 0.5 * (P.w_theta * (dx[..., :d] ** 2).sum((-1, -2)) + P.w_omega * (dx[..., d:] ** 2).sum((-1, -2))
                  + P.w_u * (U ** 2).sum((-1, -2)))
