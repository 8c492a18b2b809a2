"""Planted mistakes in a copy of the oracle must each break one of its pins (CPU only).

Each case rewrites one line of a temporary copy of ``oracle/gato_oracle.c`` the way a
plausible slip would (a dropped term, a wrong sign, a transposed operand, a wrong
index), builds it with gcc, and checks that the named pin -- which the real oracle
passes -- rejects it.  This shows the pins are sharp enough to catch such slips.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import ref
from block_tridiagonal_pcg_amd import synth
from dense_kkt import assemble, btd_dense, kkt_solve, merit_dense

ALPHAS = synth.ALPHAS.astype(np.float64)


def pin_kkt():
    """dz from the oracle equals the dense KKT LU solution (config 2, one solve)."""
    bt = synth.make_batch(2, 1)
    res = oracle.sqp_step(*synth.inputs(bt), None, 1e-12, 2000, ALPHAS, 1.0)
    d = assemble(bt, 0)
    dz, _ = kkt_solve(d["G"], d["g"], d["C"], d["c"])
    return np.linalg.norm(res["dz"][0] - dz) / np.linalg.norm(dz) < 1e-9


def pin_dense_schur():
    bt = synth.make_batch(2, 1)
    fs = oracle.form_schur(*synth.inputs(bt))
    d = assemble(bt, 0)
    Gi = np.linalg.inv(d["G"])
    S = d["C"] @ Gi @ d["C"].T
    gam = d["c"] + d["C"] @ Gi @ d["g"]
    return (np.abs(btd_dense(fs["S"][0]) - S).max() < 1e-10
            and np.abs(fs["gamma"][0].ravel() - gam).max() < 1e-10)


def pin_precond_closed_form():
    bt = synth.make_batch(2, 1)
    n, _, N, _ = bt["dims"]
    fs = oracle.form_schur(*synth.inputs(bt))
    S = btd_dense(fs["S"][0])
    Dinv = np.zeros_like(S)
    J = np.zeros_like(S)
    for k in range(N):
        sl = slice(k * n, (k + 1) * n)
        Dinv[sl, sl] = np.linalg.inv(S[sl, sl])
        J[sl, sl] = (-1) ** k * np.eye(n)
    return np.abs(btd_dense(fs["Pinv"][0]) - Dinv @ J @ S @ J @ Dinv).max() < 1e-10


def pin_library_pcg_count():
    import scipy.sparse.linalg as spla

    bt = synth.make_batch(2, 1)
    fs = oracle.form_schur(*synth.inputs(bt))
    res = oracle.pcg_solve(fs["S"], fs["Pinv"], fs["gamma"], fs["Qinv"], fs["Rinv"], bt["A"], bt["Bu"],
                           bt["q"], bt["r"], 1e-6, 200)
    cnt = [0]
    spla.cg(btd_dense(fs["S"][0]), fs["gamma"][0].ravel(), rtol=1e-6, atol=0.0,
            M=spla.aslinearoperator(btd_dense(fs["Pinv"][0])), callback=lambda x: cnt.__setitem__(0, cnt[0] + 1))
    return abs(int(res["iters"][0]) - cnt[0]) <= 1 and res["flags"][0] == 0


def pin_merit_dense():
    bt = synth.make_batch(1, 1)
    n, m, N, _ = bt["dims"]
    dz = np.random.default_rng(3).standard_normal((1, N * n + (N - 1) * m))
    res = oracle.merit_eval(*synth.inputs(bt), dz, ALPHAS, 1.3)
    d = assemble(bt, 0)
    ref_v = [merit_dense(d["G0"], d["g"], d["C"], d["c"], dz[0], a, 1.3) for a in ALPHAS]
    return np.allclose(res["merit"][0], ref_v, rtol=1e-12, atol=1e-12)


MUTATIONS = [
    ("drop B R^-1 B' from D_{k+1}", "Dk1[i] += T1[i] + T2[i];", "Dk1[i] += T1[i];", pin_dense_schur),
    ("wrong sign of S_{k,k+1}", "Sup[j * n + i] = -W[i * n + j];", "Sup[j * n + i] = W[i * n + j];",
     pin_dense_schur),
    ("drop e_k from gamma", "gk1[i] += eb[(size_t)k * n + i] - tv[i] - tv2[i];", "gk1[i] += - tv[i] - tv2[i];",
     pin_kkt),
    ("A_k instead of A_k' in the recovery",
     "mtv(n, n, A + ((size_t)b * (N - 1) + k) * nn, lam + (size_t)(k + 1) * n, t);",
     "mv(n, n, A + ((size_t)b * (N - 1) + k) * nn, lam + (size_t)(k + 1) * n, t);", pin_kkt),
    ("wrong neighbour D^-1 in the stair block",
     "mm(n, n, n, T1, Dinv + (size_t)(k + 1) * nn, T2);", "mm(n, n, n, T1, Dinv + (size_t)k * nn, T2);",
     pin_precond_closed_form),
    ("inverted beta in PCG", "double beta = eta1 / eta;", "double beta = eta / eta1;",
     pin_library_pcg_count),
    ("drop the initial-state term of the merit",
     "for (int i = 0; i < n; ++i) viol += fabs(x0[(size_t)b * n + i] - xs[i]);", "", pin_merit_dense),
    ("drop the 1/2 of the quadratic cost", "cost += dot((size_t)n, qk, xs) + 0.5 * dot((size_t)n, xs, t);",
     "cost += dot((size_t)n, qk, xs) + dot((size_t)n, xs, t);", pin_merit_dense),
]


@pytest.fixture
def swap_lib():
    saved = ref._lib

    def use(path):
        ref._lib = ref.configure(ctypes.CDLL(path))

    yield use
    ref._lib = saved


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, pin, tmp_path, swap_lib):
    oracle.load()
    assert pin(), "the real oracle must pass the pin"
    src = open(ref._SRC).read()
    assert src.count(old) == 1, "mutation anchor must be unique: %s" % old
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / ("libmut_%d.so" % abs(hash(name))))
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", so, str(mutated), "-lm"], check=True)
    swap_lib(so)
    assert not pin(), "planted mistake '%s' was not caught" % name
    os.remove(so)
