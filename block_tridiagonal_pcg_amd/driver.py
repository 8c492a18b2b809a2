"""Multi-iteration SQP driver around gato_sqp_step: the outer loop of the GATO pages'
solver (GATO paper Sec. III-IV; its docs' solve loop), on the device.

Per iteration, for every solve of the batch at once, three kernel launches:
  1. gato_chain_qp: linearise the plant (synth.Chain) about the current trajectory
     (X, U) and form the QP data Q, q, R, r, A, B, e and the initial-state defect x0;
  2. gato_sqp_step: Schur complement, PCG (warm-started from the previous
     iteration's lambda) or the direct solve, recovery, merit and step selection;
  3. gato_take_step: the selected step X += a dX, U += a dU (no step when the line
     search failed) and the damping update: a full step (a = 1) divides rho by 10,
     a shortened step keeps it, a failed line search multiplies it by 10, within
     [1e-8, 10].
The seed is the cold "hold-at-x" trajectory (every state at x_init, zero
controls), and rho starts log-spaced over 1e-8 .. 10 across the batch
(synth.chain_seed), as in the pages' rho sampling.  This module only allocates the
state and marshals the calls; the arithmetic is in the library's kernels.
"""
import numpy as np
import torch

from . import ops, synth

RHO_MIN, RHO_MAX = 1e-8, 1e1


def solve(P: synth.Chain, x_init, x_ref, rho0, N, iters, alphas=synth.ALPHAS, mu=1.0, eps=1e-6, max_iters=200,
          device="cuda", record=True, step_events=False, graph=False, on_iteration=None):
    """Run `iters` SQP iterations on the batch.  x_init, x_ref [B][n] and rho0 [B] are
    host arrays; returns the final trajectory and, with `record`, per-iteration
    history (selected step, defect, cost, rho, PCG iterations, flags) on the host.
    With `step_events`, also the device time of each gato_sqp_step (us).

    With `graph`, the first iteration runs eagerly and the second is captured in a
    HIP graph (torch.cuda.CUDAGraph) that is replayed for the rest: one iteration
    (gato_chain_qp, gato_sqp_step, gato_take_step) is then one graph launch.  The
    state (X, U, rho, lambda) lives in fixed tensors updated in place, so every replay
    continues from the previous one.  `on_iteration(k, state)` is called after each
    iteration (after a synchronisation when given)."""
    B = x_init.shape[0]
    n, m = P.n, P.m
    dims = (n, m, N, B)
    f32 = torch.float32
    prm = ops.chain_params(P)
    xi = torch.as_tensor(np.asarray(x_init), dtype=f32, device=device).contiguous()
    xr = torch.as_tensor(np.asarray(x_ref), dtype=f32, device=device).contiguous()
    X = xi[:, None, :].repeat(1, N, 1).contiguous()  # hold at x
    U = torch.zeros((B, N - 1, m), dtype=f32, device=device)
    rho = torch.as_tensor(np.asarray(rho0), dtype=f32, device=device).contiguous()
    qp = {k: torch.empty(v, dtype=f32, device=device) for k, v in ops._shapes(n, m, N, B).items()
          if k in synth.FIELDS}
    out = ops.alloc_outputs(dims, len(alphas), device=device)  # lambda starts at zero, then carries over
    ws = ops.workspace_for(dims, len(alphas), device=device)
    evs = []

    def body(events=False):
        ops.gato_chain_qp(dims, prm, X, U, xi, xr, *[qp[k] for k in synth.FIELDS])
        if events:
            evs.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
            evs[-1][0].record()
        ops.gato_sqp_step(dims, *[qp[k] for k in synth.FIELDS], rho, eps, max_iters, alphas, mu, out["lam"],
                          out["dz"], out["merit"], out["merit0"], out["best"], out["iters"], out["relres"],
                          out["flags"], workspace=ws)
        if events:
            evs[-1][1].record()
        ops.gato_take_step(dims, alphas, out["dz"], out["best"], X, U, rho, RHO_MIN, RHO_MAX)

    hist = []
    diag = {k: torch.empty_like(v) for k, v in qp.items()}

    def after(k):
        if record:
            # diagnostics at the new trajectory: its nonlinear defect (sum of |e_k| and
            # |x_init - x_0|, from the plant kernel) and its tracking cost
            ops.gato_chain_qp(dims, prm, X, U, xi, xr, *[diag[f] for f in synth.FIELDS])
            d = P.dof
            dx = X - xr[:, None, :]
            cost = 0.5 * (P.w_theta * (dx[..., :d] ** 2).sum((-1, -2)) + P.w_omega * (dx[..., d:] ** 2).sum((-1, -2))
                          + P.w_u * (U ** 2).sum((-1, -2)))
            defect = diag["e"].abs().sum((-1, -2)) + diag["x0"].abs().sum(-1)
            hist.append(dict(best=out["best"].cpu().numpy(), defect=defect.cpu().numpy(), cost=cost.cpu().numpy(),
                             rho=rho.cpu().numpy(), iters=out["iters"].cpu().numpy(),
                             flags=out["flags"].cpu().numpy()))
        if on_iteration is not None:
            torch.cuda.synchronize()
            on_iteration(k, dict(X=X, U=U, rho=rho, lam=out["lam"], best=out["best"]))

    if not graph:
        for k in range(iters):
            body(step_events)
            after(k)
    else:
        if iters >= 1:
            body()  # eager: warms the libraries up
            after(0)
        if iters >= 2:
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                body()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for k in range(1, iters):
                g.replay()
                after(k)
            e1.record()
    res = dict(X=X, U=U, lam=out["lam"], history=hist)
    if graph and iters >= 2:
        torch.cuda.synchronize()
        res["replay_us"] = 1e3 * e0.elapsed_time(e1) / (iters - 1)  # per replayed iteration
    if step_events:
        torch.cuda.synchronize()
        res["step_us"] = [1e3 * a.elapsed_time(b) for a, b in evs]
    return res
