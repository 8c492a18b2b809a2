"""GPU parity of the direct block-tridiagonal solve (gato_direct_solve) against the
fp64 oracle's block Cholesky of S, on the same seeded float32 inputs.

Tolerance: the direct solve's only error is fp32 rounding of S, gamma and the
elimination, so dz against the oracle's exact step is held to the stage-2 bar,
||dz_gpu - dz_exact|| / ||dz_exact|| <= 1e-3, on every configuration, and to 5e-5 on
the well-conditioned ones (an fp32 emulation of the same elimination gives at most
6.5e-6 there and 3e-4 on the ill-conditioned long-horizon workload).
"""
import numpy as np
import pytest
import torch

import oracle
from block_tridiagonal_pcg_amd import ops, synth
from gpu_util import gpu_direct, rel_rows

pytestmark = pytest.mark.gpu

SMALL = {1: 1, 2: 8, 3: 16, 4: 16, 5: 4}
TIGHT = {1: 5e-5, 2: 5e-5, 3: 5e-5, 4: 5e-5, 5: 1e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.load()
    oracle.load()


def _ident(*a):
    print("case:", *a, flush=True)


def _exact(bt, form):
    """The oracle's exact step: block Cholesky of S, then the recovery."""
    lam = oracle.direct_solve(form["S"], form["gamma"])["lam"]
    dz = oracle.recover(form["Qinv"], form["Rinv"], bt["A"], bt["Bu"], bt["q"], bt["r"], lam)
    return lam, dz


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_direct_parity(cid):
    B = SMALL[cid]
    _ident("direct", cid, B)
    bt = synth.make_batch(cid, B)
    form = oracle.form_schur(*synth.inputs(bt))
    g = gpu_direct(bt, form)
    lam, dz = _exact(bt, form)
    err = rel_rows(g["dz"], dz)
    print("dz rel err max %.3e median %.3e; lambda rel err max %.3e" % (err.max(), np.median(err),
                                                                        rel_rows(g["lam"], lam).max()))
    assert (g["flags"] == 0).all()
    assert err.max() <= TIGHT[cid]


@pytest.mark.parametrize("N", [1, 2, 5, 63, 64, 65, 129, 256])
def test_direct_horizons(N):
    B = 5  # not a multiple of the solves per wave: the last wave is partly empty
    _ident("direct horizon", N, B)
    bt = synth.make_batch(3, B, N=N)
    form = oracle.form_schur(*synth.inputs(bt))
    g = gpu_direct(bt, form)
    _, dz = _exact(bt, form)
    assert (g["flags"] == 0).all()
    assert rel_rows(g["dz"], dz).max() <= 5e-5


@pytest.mark.parametrize("nm", [(1, 1), (12, 6), (24, 12)])
def test_direct_other_shapes(nm):
    n, m = nm
    _ident("direct shape", n, m)
    bt = synth.make_batch(2, 3, n=n, m=m, N=9)
    form = oracle.form_schur(*synth.inputs(bt))
    g = gpu_direct(bt, form)
    _, dz = _exact(bt, form)
    assert rel_rows(g["dz"], dz).max() <= 5e-5


def test_direct_independent_of_batch_position():
    big = synth.make_batch(3, 9)
    fb = oracle.form_schur(*synth.inputs(big))
    g = gpu_direct(big, fb)
    for b in (0, 4, 8):
        one = synth.make_batch(3, 1, first=b)
        h = gpu_direct(one, oracle.form_schur(*synth.inputs(one)))
        np.testing.assert_array_equal(h["dz"][0], g["dz"][b])
        np.testing.assert_array_equal(h["lam"][0], g["lam"][b])


def test_direct_flags():
    bt = synth.make_batch(3, 4)
    form = oracle.form_schur(*synth.inputs(bt))
    bad = {k: np.array(v, copy=True) for k, v in form.items()}
    bad["S"][1] = -bad["S"][1]          # negative definite: the first pivot fails
    bad["gamma"][2, 5, 3] = np.nan      # a non-finite right-hand side
    g = gpu_direct(bt, bad, flags=np.array([0, 0, 0, 32], np.int32))
    assert g["flags"][0] == 0
    assert g["flags"][1] & ops.F_S_NOT_SPD
    assert g["flags"][2] & ops.F_NONFINITE
    assert g["flags"][3] == 32  # ORed into the bits already there
