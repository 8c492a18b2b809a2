"""Analytic nonlinear plant for the multi-iteration SQP driver: a chain of coupled,
damped pendulums (a synthetic stand-in for the robot models the GATO pages linearise
with GRiD, which are not reproduced here).

State x = [theta (d), omega (d)], control u (d joint torques): n = 2d, m = d, so
d = 7 gives the 7-DoF-arm shape (14, 7).  Explicit Euler with step h:
    theta' = theta + h omega
    omega' = omega + h (-a sin(theta) - c omega + kappa L theta + u)
with L the path-graph Laplacian over the joints (free ends).  The cost tracks a
target angle vector: 1/2 (x - x_ref)' W (x - x_ref) + 1/2 u' Rw u, with diagonal W, Rw.

Functions work on batched arrays X [B][N][n], U [B][N-1][m] that are either numpy
(fp64, the reference driver) or torch (the device driver).  Nothing here is part of
the method (the formation, PCG or merit): it only supplies each SQP iteration's QP
data Q, q, R, r, A, B, e and the initial-state defect (GATO paper Sec. II, Step 1).
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Chain:
    dof: int
    h: float = 0.02
    a: float = 9.81
    c: float = 0.5
    kappa: float = 2.0
    w_theta: float = 10.0
    w_omega: float = 0.1
    w_u: float = 0.01

    @property
    def n(self):
        return 2 * self.dof

    @property
    def m(self):
        return self.dof


def _torch(x):
    return not isinstance(x, np.ndarray)


def _lib(x):
    if _torch(x):
        import torch

        return torch
    return np


def _cat(parts):
    if _torch(parts[0]):
        import torch

        return torch.cat(parts, -1)
    return np.concatenate(parts, -1)


_DEVICE_CONSTS = {}


def _const(x, a):
    """Constant array `a` (numpy) with x's dtype and device.  Device copies are made
    once per (value, dtype, device) and reused, so that the plant's functions launch
    no host-to-device copy after their first call (and can be captured in a graph)."""
    if _torch(x):
        import torch

        a = np.ascontiguousarray(a)
        key = (a.tobytes(), a.shape, str(x.dtype), str(x.device))
        t = _DEVICE_CONSTS.get(key)
        if t is None:
            t = torch.as_tensor(a, dtype=x.dtype, device=x.device)
            _DEVICE_CONSTS[key] = t
        return t
    return np.asarray(a, dtype=x.dtype)


def _tile(x, small, shape):
    """The constant `small` (numpy) repeated to `shape`, as a new array like x."""
    if _torch(x):
        return _const(x, small).expand(shape).contiguous()
    return np.broadcast_to(np.asarray(small, dtype=x.dtype), shape).copy()


def laplacian_matrix(d):
    L = -2.0 * np.eye(d)
    for j in range(d - 1):
        L[j, j + 1] = L[j + 1, j] = 1.0
    L[0, 0] += 1.0
    L[d - 1, d - 1] += 1.0
    return L


def step(P: Chain, X, U):
    """f(x_k, u_k) for every knot that has a control: [B][N-1][n]."""
    xp = _lib(X)
    d = P.dof
    th, om = X[..., :-1, :d], X[..., :-1, d:]
    acc = -P.a * xp.sin(th) - P.c * om + P.kappa * (th @ _const(X, laplacian_matrix(d))) + U
    return _cat([th + P.h * om, om + P.h * acc])


def linearize(P: Chain, X, U):
    """A_k = df/dx, B_k = df/du at (x_k, u_k), and the defects e_k = f(x_k, u_k) - x_{k+1}."""
    xp = _lib(X)
    d, n = P.dof, P.n
    th = X[..., :-1, :d]
    shape = tuple(th.shape[:-1])
    eye = _const(X, np.eye(d))
    A = xp.zeros(shape + (n, n), dtype=X.dtype) if not _torch(X) else xp.zeros(shape + (n, n), dtype=X.dtype,
                                                                                 device=X.device)
    Bu = xp.zeros(shape + (n, d), dtype=X.dtype) if not _torch(X) else xp.zeros(shape + (n, d), dtype=X.dtype,
                                                                                  device=X.device)
    cos_diag = xp.cos(th)[..., :, None] * eye  # diag(cos theta) per knot
    A[..., :d, :d] = eye
    A[..., :d, d:] = P.h * eye
    A[..., d:, :d] = P.h * (-P.a * cos_diag + P.kappa * _const(X, laplacian_matrix(d)))
    A[..., d:, d:] = (1.0 - P.h * P.c) * eye
    Bu[..., d:, :] = P.h * eye
    e = step(P, X, U) - X[..., 1:, :]
    return A, Bu, e


def cost_terms(P: Chain, X, U, x_ref):
    """Q_k = W, q_k = W (x_k - x_ref), R_k = Rw, r_k = Rw u_k for the tracking cost."""
    d, n = P.dof, P.n
    w = np.concatenate([np.full(d, P.w_theta), np.full(d, P.w_omega)])
    Q = _tile(X, np.diag(w), tuple(X.shape[:-1]) + (n, n))
    R = _tile(X, P.w_u * np.eye(d), tuple(U.shape[:-1]) + (d, d))
    q = (X - x_ref[:, None, :]) * _const(X, w)
    r = P.w_u * U
    return Q, q, R, r


def defect(P: Chain, X, U, x_init):
    """Nonlinear constraint violation per solve: sum_k ||f(x_k,u_k) - x_{k+1}||_1 + ||x_init - x_0||_1."""
    e = step(P, X, U) - X[..., 1:, :]
    return abs(e).sum((-1, -2)) + abs(x_init - X[..., 0, :]).sum(-1)


def cost(P: Chain, X, U, x_ref):
    d = P.dof
    dx = X - x_ref[:, None, :]
    return 0.5 * (P.w_theta * (dx[..., :d] ** 2).sum((-1, -2)) + P.w_omega * (dx[..., d:] ** 2).sum((-1, -2))
                  + P.w_u * (U ** 2).sum((-1, -2)))


def seed(P: Chain, B: int, first: int = 0):
    """Per-solve initial states and targets (fp64 numpy; solve b is the same for every
    B): angles and rates drawn small, target angles in [-0.6, 0.6] rad; and the
    starting damping rho, log-spaced over 1e-8 .. 1e1 across the batch."""
    x_init = np.zeros((B, P.n))
    x_ref = np.zeros((B, P.n))
    for j in range(B):
        rng = np.random.default_rng(np.random.SeedSequence([71, first + j]))
        x_init[j, :P.dof] = rng.uniform(-0.3, 0.3, P.dof)
        x_init[j, P.dof:] = rng.uniform(-0.2, 0.2, P.dof)
        x_ref[j, :P.dof] = rng.uniform(-0.6, 0.6, P.dof)
    rho = np.logspace(-8, 1, B) if B > 1 else np.array([1e-4])
    return x_init, x_ref, rho
