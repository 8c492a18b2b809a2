"""Reference for the multi-iteration SQP driver: the same outer loop as the device
driver, in fp64 numpy around the oracle's sqp_step.  Test infrastructure only.

Per iteration: linearise the plant about (X, U) (plant_ref, this package's fp64 plant;
its parameters come from the shared input module), one oracle sqp_step warm-started
from the previous lambda, the step X += a dX,
U += a dU with the selected step size a (none when the line search failed), and
the damping update: a full step divides rho by 10, a shortened one keeps it, a
failed line search multiplies it by 10, within [1e-8, 10].
"""
import numpy as np

from . import plant_ref as plant
from .ref import sqp_step


def solve(P, x_init, x_ref, rho0, N, iters, alphas, mu=1.0, eps=1e-6, max_iters=200):
    B = x_init.shape[0]
    n, m = P.n, P.m
    X = np.repeat(np.asarray(x_init, np.float64)[:, None, :], N, axis=1)
    U = np.zeros((B, N - 1, m))
    rho = np.asarray(rho0, np.float64).copy()
    al = np.asarray(alphas, np.float64)
    lam = np.zeros((B, N, n))
    hist = []
    for _ in range(iters):
        A, Bu, e = plant.linearize(P, X, U)
        Q, q, R, r = plant.cost_terms(P, X, U, x_ref)
        x0 = x_init - X[:, 0]
        res = sqp_step(Q, q, R, r, A, Bu, e, x0, rho, eps, max_iters, al, mu, lambda0=lam)
        lam = res["lam"]
        best = res["best"]
        a = np.where(best >= 0, al[np.maximum(best, 0)], 0.0)
        dz = np.concatenate([res["dz"], np.zeros((B, m))], -1).reshape(B, N, n + m)
        X = X + a[:, None, None] * dz[..., :n]
        U = U + a[:, None, None] * dz[:, :N - 1, n:]
        for b in range(B):
            if best[b] == 0:
                rho[b] = max(rho[b] / 10.0, 1e-8)
            elif best[b] < 0:
                rho[b] = min(rho[b] * 10.0, 10.0)
        hist.append(dict(best=best.copy(), merit=res["merit"].copy(), merit0=res["merit0"].copy(),
                         defect=plant.defect(P, X, U, x_init), cost=plant.cost(P, X, U, x_ref), rho=rho.copy(),
                         iters=res["iters"].copy(), flags=res["flags"].copy()))
    return dict(X=X, U=U, lam=lam, history=hist)
