"""Shapes without kernels of their own: gato_sqp_step solves them inside the smallest
compiled shape that holds them (identity rows and columns in Q_k and R_k, zeros in A_k,
B_k, q, r, e and x0), on the fused path and beyond it, against the fp64 oracle on the
original, unpadded problem.  Also the widest compiled shape, (28, 14), natively."""
import numpy as np
import pytest
import torch

import oracle
from block_tridiagonal_pcg_amd import ops, synth
from gpu_util import ALPHAS, gpu_sqp, merit_rel, rel_rows, select

pytestmark = pytest.mark.gpu
A64 = ALPHAS.astype(np.float64)

# (generators of workload, n, m, N, B): the shape it runs as is in the comment
CASES = [
    (2, 10, 5, 32, 8),    # (12, 6), fused (dense Q)
    (3, 10, 5, 100, 4),   # (12, 6), long horizon (cyclic reduction)
    (1, 3, 1, 8, 2),      # (4, 2), fused
    (4, 18, 9, 16, 8),    # (24, 12), fused, 32-lane groups
    (4, 16, 8, 40, 3),    # (24, 12), long horizon
    (4, 26, 13, 12, 4),   # (28, 14), fused
    (4, 28, 14, 16, 4),   # (28, 14) itself, fused
    (4, 28, 14, 40, 3),   # (28, 14) itself, long horizon
    (3, 13, 7, 64, 4),    # (14, 7), fused at the full horizon
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.load()
    oracle.load()


@pytest.mark.parametrize("cid,n,m,N,B", CASES, ids=["n%dm%dN%dB%d" % c[1:] for c in CASES])
def test_step_on_other_shapes(cid, n, m, N, B):
    print("case: shape", cid, n, m, N, B, flush=True)
    bt = synth.make_batch(cid, B, n=n, m=m, N=N)
    native = (n, m) in ((14, 7), (12, 6), (24, 12), (4, 2), (1, 1), (28, 14))
    assert ops.gato_shape_supported(n, m, N) == (1 if native else 2)
    g = gpu_sqp(bt, 1e-6, 400)
    ins = synth.inputs(bt)
    fused = ops.gato_step_solver(bt["dims"]) == ops.SOLVER_FUSED_PCG
    if fused:
        o = oracle.sqp_step(*ins, None, 1e-6, 400, A64, 1.0)
        ref_lam = o["lam"]
    else:
        f = oracle.form_schur(*ins)
        ref_lam = oracle.direct_solve(f["S"], f["gamma"])["lam"]
        o = {"dz": oracle.recover(f["Qinv"], f["Rinv"], bt["A"], bt["Bu"], bt["q"], bt["r"], ref_lam),
             "flags": f["flags"]}
    err = rel_rows(g["dz"], o["dz"])
    lerr = rel_rows(g["lam"], ref_lam)
    print("dz rel err max %.3e, lambda %.3e, iters %s" % (err.max(), lerr.max(), g["iters"].tolist()))
    assert err.max() <= 1e-3 and lerr.max() <= 1e-3
    assert ((g["flags"] & ~ops.F_LS_FAILED) == (o["flags"] & ~ops.F_LS_FAILED)).all()
    om = oracle.merit_eval(*ins, g["dz"].astype(np.float64), A64, 1.0)
    assert merit_rel(g["merit"], om).max() <= 1e-4
    np.testing.assert_array_equal(g["best"], select(g["merit"], g["merit0"]))
    if fused:
        assert np.abs(g["iters"] - o["iters"]).max() <= 2
    else:
        assert (g["iters"] == 0).all()


def test_padded_step_warm_start_and_noalloc():
    """A padded shape takes lambda's input (the warm start) through the padding, and the
    allocation-free entry point gives the workspace call's bits."""
    bt = synth.make_batch(2, 4, n=10, m=5, N=32)
    dims = bt["dims"]
    f = oracle.form_schur(*synth.inputs(bt))
    exact = oracle.direct_solve(f["S"], f["gamma"])["lam"]
    warm = gpu_sqp(bt, 1e-6, 400, lambda0=exact)
    assert (warm["iters"] <= 1).all()
    ref = gpu_sqp(bt, 1e-6, 400)
    dev = ops.to_device(bt)
    out = ops.alloc_outputs(dims, 8)
    ops.gato_sqp_step_noalloc(dims, *[dev[k] for k in synth.FIELDS], None, 1e-6, 400, ALPHAS, 1.0,
                              *[out[k] for k in ("lam", "dz", "merit", "merit0", "best", "iters", "relres", "flags")])
    torch.cuda.synchronize()
    for k in ("lam", "dz", "merit", "merit0", "best", "iters", "relres", "flags"):
        np.testing.assert_array_equal(out[k].cpu().numpy(), ref[k], err_msg=k)
