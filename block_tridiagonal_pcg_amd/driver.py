"""Multi-iteration SQP driver around gato_sqp_step: the outer loop of the GATO pages'
solver (GATO paper Sec. III-IV; its docs' solve loop), on the device.

Per iteration, for every solve of the batch at once:
  1. linearise the plant about the current trajectory (X, U) and form the QP data
     Q, q, R, r, A, B, e and the initial-state defect x0 (block_tridiagonal_pcg_amd.plant);
  2. one gato_sqp_step: Schur complement, PCG (warm-started from the previous
     iteration's lambda) or the direct solve, recovery, merit and step selection;
  3. take the selected step, X += a dX and U += a dU (no step when the line search
     failed);
  4. update the damping rho from the line-search outcome: a full step (a = 1)
     divides rho by 10, a shortened step keeps it, a failed line search
     multiplies it by 10, within [1e-8, 10].
The seed is the cold "hold-at-x" trajectory (every state at x_init, zero
controls), and rho starts log-spaced over 1e-8 .. 10 across the batch
(plant.seed), as in the pages' rho sampling.
"""
import numpy as np
import torch

from . import ops, plant, synth

RHO_MIN, RHO_MAX = 1e-8, 1e1


def split_dz(dz, n, m, N):
    """dz [B][N n + (N-1) m] (dx_0, du_0, ..., dx_{N-1}) -> dX [B][N][n], dU [B][N-1][m]."""
    B = dz.shape[0]
    full = torch.cat([dz, dz.new_zeros((B, m))], -1).view(B, N, n + m)
    return full[..., :n], full[:, :N - 1, n:]


def update_rho(rho, best):
    full = best == 0
    failed = best < 0
    rho = torch.where(full, torch.clamp(rho / 10.0, min=RHO_MIN), rho)
    return torch.where(failed, torch.clamp(rho * 10.0, max=RHO_MAX), rho)


def solve(P: plant.Chain, x_init, x_ref, rho0, N, iters, alphas=synth.ALPHAS, mu=1.0, eps=1e-6, max_iters=200,
          device="cuda", record=True, step_events=False, graph=False, on_iteration=None):
    """Run `iters` SQP iterations on the batch.  x_init, x_ref [B][n] and rho0 [B] are
    host arrays; returns the final trajectory and, with `record`, per-iteration
    history (selected step, defect, cost, rho, PCG iterations, flags) on the host.
    With `step_events`, also the device time of each gato_sqp_step (us).

    With `graph`, the first iteration runs eagerly and the second is captured in a
    HIP graph (torch.cuda.CUDAGraph) that is replayed for the rest: one iteration
    (linearisation, cost terms, gato_sqp_step, the step and the damping update) is
    then one graph launch instead of some forty small kernel launches.  The state
    (X, U, rho, lambda) lives in fixed tensors updated in place, so every replay
    continues from the previous one.  `on_iteration(k, state)` is called after each
    iteration (after a synchronisation when given)."""
    B = x_init.shape[0]
    n, m = P.n, P.m
    dims = (n, m, N, B)
    f32 = torch.float32
    xi = torch.as_tensor(np.asarray(x_init), dtype=f32, device=device)
    xr = torch.as_tensor(np.asarray(x_ref), dtype=f32, device=device)
    X = xi[:, None, :].repeat(1, N, 1).contiguous()  # hold at x
    U = torch.zeros((B, N - 1, m), dtype=f32, device=device)
    rho = torch.as_tensor(np.asarray(rho0), dtype=f32, device=device).contiguous()
    al = torch.as_tensor(np.asarray(alphas), dtype=f32, device=device)
    out = ops.alloc_outputs(dims, len(alphas), device=device)  # lambda starts at zero, then carries over
    ws = ops.workspace_for(dims, len(alphas), device=device)
    zero = torch.zeros_like(rho)
    evs = []

    def body(events=False):
        A, Bu, e = plant.linearize(P, X, U)
        Q, q, R, r = plant.cost_terms(P, X, U, xr)
        x0 = (xi - X[:, 0]).contiguous()
        if events:
            evs.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
            evs[-1][0].record()
        ops.gato_sqp_step(dims, Q, q, R, r, A, Bu, e, x0, rho, eps, max_iters, alphas, mu, out["lam"], out["dz"],
                          out["merit"], out["merit0"], out["best"], out["iters"], out["relres"], out["flags"],
                          workspace=ws)
        if events:
            evs[-1][1].record()
        best = out["best"].long()
        a = torch.where(best >= 0, al[best.clamp(min=0)], zero)
        dX, dU = split_dz(out["dz"], n, m, N)
        X.add_(a[:, None, None] * dX)
        U.add_(a[:, None, None] * dU)
        rho.copy_(update_rho(rho, best))

    hist = []

    def after(k):
        if record:
            hist.append(dict(best=out["best"].cpu().numpy(), defect=plant.defect(P, X, U, xi).cpu().numpy(),
                             cost=plant.cost(P, X, U, xr).cpu().numpy(), rho=rho.cpu().numpy(),
                             iters=out["iters"].cpu().numpy(), flags=out["flags"].cpu().numpy()))
        if on_iteration is not None:
            torch.cuda.synchronize()
            on_iteration(k, dict(X=X, U=U, rho=rho, lam=out["lam"], best=out["best"]))

    if not graph:
        for k in range(iters):
            body(step_events)
            after(k)
    else:
        if iters >= 1:
            body()  # eager: also allocates the plant's device constants and warms the libraries up
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
