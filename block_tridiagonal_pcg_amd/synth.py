"""Seeded synthetic LQ subproblems shaped like the GATO pages' workloads.

This module only draws inputs.  It holds none of the method's arithmetic, and
it is the one piece of code that both the HIP path's tests/benchmark and the
fp64 oracle's tests use.

The pages measure on robot problems (Indy7, iiwa14, Go2 with GRiD dynamics)
whose models are not available, so the batches below stand in for them with
the same shapes: n = 2*DoF states, m = DoF controls, N knot points, B solves.

Recipe, per solve b of configuration c (so that solve b is the same for any
batch size B -- the prefix property):
  rng = numpy Generator(PCG64(SeedSequence([c, b])));
  draw order: Q_k for k < N; then for each k < N-1: A_k, B_k, R_k; then
  q (N x n), r (N-1 x m), e (N-1 x n), x0 (n);
  A_k = M * rho_A / max|eig(M)| with M = I + 0.1 * N(0,1)   (spectral radius rho_A)
  B_k ~ N(0, 0.1)  (standard deviation 0.1)
  Q_k: diag U[1,10] | L L' + I with L ~ N(0, 0.3) | diag 10^U[-3,3]
  R_k: diag U[r_lo, 1]
  q, r, x0 ~ N(0,1);  e ~ N(0, s_e)
Everything is drawn in float64 and rounded once to float32; the oracle upcasts
those same float32 values, so a comparison measures solver error only.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    n: int
    m: int
    N: int
    batches: tuple
    rho_A: float
    q_kind: str  # "diag" | "dense" | "logdiag"
    r_lo: float
    e_std: float


CONFIGS = {
    1: Config(1, "single LQ solve n4 m2 N8", 4, 2, 8, (1,), 0.95, "diag", 0.1, 1.0),
    2: Config(2, "6-DoF-arm-shaped n12 m6 N32", 12, 6, 32, (1, 8, 16), 0.95, "dense", 0.1, 1.0),
    3: Config(3, "7-DoF-arm-shaped n14 m7 N64", 14, 7, 64, (1, 8, 16, 64, 128), 0.95, "diag", 0.1, 0.01),
    4: Config(4, "legged-robot-shaped n24 m12 N16", 24, 12, 16, (16, 64, 256), 0.98, "diag", 0.01, 1.0),
    5: Config(5, "ill-conditioned long-horizon n14 m7 N128", 14, 7, 128, (512,), 0.999, "logdiag", 0.1, 1.0),
}

ALPHAS = np.array([2.0 ** -i for i in range(8)], dtype=np.float32)

FIELDS = ("Q", "q", "R", "r", "A", "Bu", "e", "x0")


def _one_solve(cfg: Config, b: int, n: int, m: int, N: int):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.cid, b])))
    Q = np.empty((N, n, n))
    for k in range(N):
        if cfg.q_kind == "diag":
            Q[k] = np.diag(rng.uniform(1.0, 10.0, n))
        elif cfg.q_kind == "dense":
            L = rng.normal(0.0, 0.3, (n, n))
            Q[k] = L @ L.T + np.eye(n)
        elif cfg.q_kind == "logdiag":
            Q[k] = np.diag(10.0 ** rng.uniform(-3.0, 3.0, n))
        else:
            raise ValueError(cfg.q_kind)
    A = np.empty((max(N - 1, 0), n, n))
    Bu = np.empty((max(N - 1, 0), n, m))
    R = np.empty((max(N - 1, 0), m, m))
    for k in range(N - 1):
        M = np.eye(n) + 0.1 * rng.standard_normal((n, n))
        A[k] = M * (cfg.rho_A / np.max(np.abs(np.linalg.eigvals(M))))
        Bu[k] = rng.normal(0.0, 0.1, (n, m))
        R[k] = np.diag(rng.uniform(cfg.r_lo, 1.0, m))
    q = rng.standard_normal((N, n))
    r = rng.standard_normal((max(N - 1, 0), m))
    e = rng.normal(0.0, cfg.e_std, (max(N - 1, 0), n))
    x0 = rng.standard_normal(n)
    return dict(Q=Q, q=q, R=R, r=r, A=A, Bu=Bu, e=e, x0=x0)


def make_batch(cid: int, B: int, *, n: int | None = None, m: int | None = None,
               N: int | None = None, first: int = 0) -> dict:
    """float32 arrays for solves first..first+B-1 of configuration ``cid``.

    ``n``, ``m``, ``N`` override the configuration's sizes (same generators)
    for edge-case tests (N = 1, ragged horizons, other state sizes).
    """
    cfg = CONFIGS[cid]
    n = cfg.n if n is None else n
    m = cfg.m if m is None else m
    N = cfg.N if N is None else N
    per = [_one_solve(cfg, first + b, n, m, N) for b in range(B)]
    out = {}
    for f in FIELDS:
        out[f] = np.ascontiguousarray(np.stack([p[f] for p in per]).astype(np.float32))
    out["dims"] = (n, m, N, B)
    return out


def inputs(batch: dict):
    """The eight problem arrays in the C-ABI argument order."""
    return [batch[f] for f in FIELDS]


# ---------------------------------------------------------------- the SQP driver's plant


@dataclass(frozen=True)
class Chain:
    """Parameters of the analytic plant the multi-iteration SQP driver runs on (a
    synthetic stand-in for the robot models the pages linearise with GRiD): a chain of
    `dof` coupled, damped pendulums, state x = [theta, omega], control u (torques), so
    n = 2 dof and m = dof; explicit Euler with step h,
        theta' = theta + h omega,
        omega' = omega + h (-a sin(theta) - c omega + kappa L theta + u),
    L the path-graph Laplacian over the joints (free ends); the cost tracks a target,
        1/2 (x - x_ref)' diag(w_theta, w_omega) (x - x_ref) + 1/2 w_u u'u.
    The arithmetic lives on each side of its own: the device driver's kernels
    (gato_chain_qp) and the reference driver's fp64 plant (oracle)."""
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


def chain_seed(P: Chain, B: int, first: int = 0):
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
