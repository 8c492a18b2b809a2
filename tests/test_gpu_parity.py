"""GPU parity: every C-ABI call against the fp64 oracle on the same seeded inputs.

Tolerances (the GPU computes in fp32):
  stage 1  S, gamma, Q~^-1, R^-1: <= 1e-5 relative Frobenius per solve; Phi^-1: <= 1e-4
           (fp32 entries carry ~6e-8 relative rounding; Gauss-Jordan inverses of blocks
           with condition numbers up to ~5e5 lose a few more digits);
  stage 2  ||dz_gpu - dz_oracle|| / ||dz_oracle|| <= 1e-3 at a PCG exit tolerance of 1e-6;
  stage 3  merit <= 1e-4 relative, with the denominator max(|M_oracle(a)|, M0), when both
           sides evaluate the same step.
Integer outputs decided by floats (the selected step) are compared with the selection
rule applied to the GPU's own fp32 merits; flags other than the line-search bit must match.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from block_tridiagonal_pcg_amd import ops, synth
from gpu_util import (ALPHAS, CAPS, btd_min_pivot_eig, btd_relres, gpu_form, gpu_merit, gpu_pcg, gpu_sqp,
                      merit_rel, rel_rows, select)

pytestmark = pytest.mark.gpu

A64 = ALPHAS.astype(np.float64)
SMALL = {1: 1, 2: 8, 3: 16, 4: 16, 5: 4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.load()
    oracle.load()


def _batch(cid, B, **kw):
    return synth.make_batch(cid, B, **kw)


def _ident(*a):
    print("case:", *a, flush=True)


def _direct_path(bt):
    """gato_sqp_step solves S lambda = gamma directly when a workgroup cannot hold the horizon."""
    n, _, N, _ = bt["dims"]
    return N > (64 if n <= 16 else 16)


# ---------------------------------------------------------------- stage 1


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_form_parity(cid):
    B = SMALL[cid]
    _ident("form", cid, B)
    bt = _batch(cid, B)
    rho = np.linspace(0.0, 0.3, B)
    g = gpu_form(bt, rho=rho)
    o = oracle.form_schur(*synth.inputs(bt), rho=rho.astype(np.float32))
    assert rel_rows(g["S"], o["S"]).max() <= 1e-5
    assert rel_rows(g["gamma"], o["gamma"]).max() <= 1e-5
    assert rel_rows(g["Qinv"], o["Qinv"]).max() <= 1e-5
    if bt["dims"][2] > 1:
        assert rel_rows(g["Rinv"], o["Rinv"]).max() <= 1e-5
    assert rel_rows(g["Pinv"], o["Pinv"]).max() <= 1e-4
    np.testing.assert_array_equal(g["flags"], o["flags"])
    # out-of-range blocks are written as zeros
    assert np.all(g["S"][:, 0, 0] == 0) and np.all(g["S"][:, -1, 2] == 0)
    assert np.all(g["Pinv"][:, 0, 0] == 0) and np.all(g["Pinv"][:, -1, 2] == 0)


@pytest.mark.parametrize("cid", [2, 4])  # 16-lane groups (n = 12) and 32-lane groups (n = 24)
def test_inverses_keep_their_accuracy_at_large_pivots(cid):
    """Q and R scaled by 1e3: the Gauss-Jordan inverses scale each row by its pivot's
    reciprocal once, at the end, so the inverses, S and Phi^-1 keep fp32 accuracy
    (~1e-7) however large the pivots.  Scaling the pivot row inside each step with the
    multiplier 1/piv - 1 rounds that multiplier in absolute terms; with dense Q at this
    scale that cost ~1.3e-5 (16-lane groups)."""
    _ident("inverses at large pivots", cid)
    bt = _batch(cid, 16)
    bt["Q"] = (bt["Q"] * np.float32(1e3)).astype(np.float32)
    bt["R"] = (bt["R"] * np.float32(1e3)).astype(np.float32)
    g = gpu_form(bt)
    o = oracle.form_schur(*synth.inputs(bt))
    errs = {k: rel_rows(g[k], o[k]).max() for k in ("Qinv", "Rinv", "S", "gamma", "Pinv")}
    print(errs)
    assert max(errs.values()) <= 1e-6
    assert (g["flags"] == 0).all()


def test_stair_preconditioner_on_the_ill_conditioned_workload():
    """Phi^-1 from gato_form_schur on all 512 solves of workload 5 against the oracle's,
    and its definiteness (the sign of the smallest eigenvalue over the block LDL' pivots
    of its symmetric part, in fp64).  The exact Phi^-1 rounded to fp32 is definite on
    every solve, but the fp32 inversions of the D_k (condition up to ~5e5) leave Phi^-1
    within ~5e-5 of the oracle's, enough to make it indefinite on a few solves; PCG
    therefore switches to the factored form there (tested above)."""
    bt = _batch(5, 512)
    _ident("Phi^-1 on workload 5", bt["dims"])
    g = gpu_form(bt)
    o = oracle.form_schur(*synth.inputs(bt))
    err = rel_rows(g["Pinv"], o["Pinv"])
    derr = rel_rows(g["Pinv"][:, :, 1], o["Pinv"][:, :, 1])
    ev = btd_min_pivot_eig(g["Pinv"])
    ev32 = btd_min_pivot_eig(o["Pinv"].astype(np.float32))
    print("Phi^-1 rel err max %.3e median %.3e; D^-1 max %.3e; indefinite on the GPU: %d (%s); "
          "exact rounded to fp32: %d" % (err.max(), np.median(err), derr.max(), (ev <= 0).sum(),
                                         np.nonzero(ev <= 0)[0].tolist(), (ev32 <= 0).sum()))
    assert err.max() <= 1e-4 and derr.max() <= 1e-4
    assert (ev32 > 0).all()
    assert (ev <= 0).sum() <= 16
    assert rel_rows(g["S"], o["S"]).max() <= 1e-6


@pytest.mark.parametrize("cid", [2, 4])  # 16-lane groups (n = 12) and 32-lane groups (n = 24)
def test_form_flags_match_oracle(cid):
    _ident("form flags", cid)
    bt = _batch(cid, 4)
    n = bt["dims"][0]
    bt["Q"][1, 5] = -np.eye(n, dtype=np.float32)
    bt["R"][2, 7] = -np.eye(bt["dims"][1], dtype=np.float32)
    bt["Q"][3, -1] = -1e-3 * np.eye(n, dtype=np.float32)
    g = gpu_form(bt)
    o = oracle.form_schur(*synth.inputs(bt))
    # Once a pivot fails the two sides carry different garbage downstream (the oracle's
    # Cholesky yields NaN, Gauss-Jordan a finite flagged inverse), so the S bit of a solve
    # whose Q or R failed is not compared.
    qr = ops.F_Q_NOT_SPD | ops.F_R_NOT_SPD
    np.testing.assert_array_equal(g["flags"] & qr, o["flags"] & qr)
    clean = (o["flags"] & qr) == 0
    np.testing.assert_array_equal(g["flags"][clean], o["flags"][clean])
    assert g["flags"][0] == 0 and g["flags"][1] & ops.F_Q_NOT_SPD and g["flags"][2] & ops.F_R_NOT_SPD
    assert g["flags"][3] & ops.F_S_NOT_SPD


# ---------------------------------------------------------------- stage 2


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_pcg_parity(cid):
    B = SMALL[cid]
    _ident("pcg", cid, B)
    bt = _batch(cid, B)
    o_form = oracle.form_schur(*synth.inputs(bt))
    g = gpu_pcg(bt, o_form, 1e-6, CAPS[cid])
    o = oracle.pcg_solve(o_form["S"], o_form["Pinv"], o_form["gamma"], o_form["Qinv"], o_form["Rinv"], bt["A"],
                         bt["Bu"], bt["q"], bt["r"], 1e-6, CAPS[cid])
    err = rel_rows(g["dz"], o["dz"])
    print("dz rel err max %.3e; iters gpu %s oracle %s" % (err.max(), g["iters"].tolist(), o["iters"].tolist()))
    assert err.max() <= 1e-3
    assert (g["flags"] == 0).all() and (o["flags"] == 0).all()
    assert (g["relres"] <= 1e-6).all()
    if cid != 5:
        assert np.abs(g["iters"] - o["iters"]).max() <= 2


@pytest.mark.parametrize("cid,N", [(3, 65), (3, 100), (2, 100), (1, 90), (3, 129), (3, 200), (3, 256), (4, 17),
                                   (4, 40), (4, 64)])
def test_pcg_streamed_horizons(cid, N):
    """gato_pcg_solve beyond one workgroup's horizon (several knots per lane group, rows
    re-read per product): up to 256 knots for 16-lane groups and 64 for 32-lane ones,
    including ragged last chunks; with two knots per 16-lane group (N <= 128) S's
    diagonal blocks and D^-1 stay on chip, for every shape that kernel has."""
    B = 2
    _ident("pcg streamed", cid, N, B)
    bt = _batch(cid, B, N=N)
    o_form = oracle.form_schur(*synth.inputs(bt))
    g = gpu_pcg(bt, o_form, 1e-6, 400)
    o = oracle.pcg_solve(o_form["S"], o_form["Pinv"], o_form["gamma"], o_form["Qinv"], o_form["Rinv"], bt["A"],
                         bt["Bu"], bt["q"], bt["r"], 1e-6, 400)
    assert (g["flags"] == 0).all() and (o["flags"] == 0).all()
    assert (g["relres"] <= 1e-6).all()
    assert rel_rows(g["dz"], o["dz"]).max() <= 1e-3
    assert np.abs(g["iters"] - o["iters"]).max() <= 2


def test_pcg_streamed_converges_where_the_assembled_preconditioner_is_indefinite():
    """gato_pcg_solve on the GPU-formed system of the ill-conditioned long-horizon
    workload (N = 128: two knots per lane group, rows streamed).  For solves 188, 190,
    240, 310 and 316 of its 512-solve batch the assembled fp32 Phi^-1 is indefinite or
    nearly so (cond ~1e10); applied in its factored form the preconditioner stays
    definite, and every solve converges within 1.3x the oracle's iterations with dz
    within 1e-3 of the oracle's PCG step."""
    full = synth.make_batch(5, 512)
    idx = np.array([188, 190, 240, 310, 316, 0, 1])
    n, m, N, _ = full["dims"]
    bt = {k: (v[idx] if k != "dims" else (n, m, N, len(idx))) for k, v in full.items()}
    dims = bt["dims"]
    _ident("pcg streamed, ill-conditioned solves", idx)
    dev = ops.to_device(bt)
    st = ops.alloc_outputs(dims, 8)
    ops.gato_form_schur(dims, *[dev[f] for f in synth.FIELDS], None, st["S"], st["Pinv"], st["gamma"],
                        st["Qinv"], st["Rinv"], st["flags"])
    st["lam"].zero_()
    ops.gato_pcg_solve(dims, st["S"], st["Pinv"], st["gamma"], st["Qinv"], st["Rinv"], dev["A"], dev["Bu"],
                       dev["q"], dev["r"], 1e-6, 2000, st["lam"], st["dz"], st["iters"], st["relres"], st["flags"])
    torch.cuda.synchronize()
    o_form = oracle.form_schur(*synth.inputs(bt))
    o = oracle.pcg_solve(o_form["S"], o_form["Pinv"], o_form["gamma"], o_form["Qinv"], o_form["Rinv"], bt["A"],
                         bt["Bu"], bt["q"], bt["r"], 1e-6, 2000)
    it, fl = st["iters"].cpu().numpy(), st["flags"].cpu().numpy()
    print("iters", it, "oracle", o["iters"])
    assert (fl == 0).all() and (o["flags"] == 0).all()
    assert (it <= 1.3 * o["iters"]).all()
    assert rel_rows(st["dz"].cpu().numpy(), o["dz"]).max() <= 1e-3


def test_pcg_iterations_match_the_oracle_on_the_ill_conditioned_workload():
    """Every solve of the ill-conditioned long-horizon workload (B = 512, N = 128, cap
    2000): gato_form_schur, then gato_pcg_solve (two knots per lane group, Phi^-1 in
    factored form) against the oracle's PCG on its own fp64 formation.  The two count
    S-products under the same exit test; the fp32 iteration differs from the fp64 one
    by rounding, so the counts are compared as a ratio: no solve at the cap, each
    within [0.75, 1.5] of the oracle's, the median within [0.9, 1.15]; dz within the
    1e-3 bar of the oracle's PCG step."""
    bt = _batch(5, 512)
    dims = bt["dims"]
    _ident("pcg iterations vs oracle, workload 5", dims)
    dev = ops.to_device(bt)
    st = ops.alloc_outputs(dims, 8)
    ops.gato_form_schur(dims, *[dev[f] for f in synth.FIELDS], None, st["S"], st["Pinv"], st["gamma"],
                        st["Qinv"], st["Rinv"], st["flags"])
    st["lam"].zero_()
    ops.gato_pcg_solve(dims, st["S"], st["Pinv"], st["gamma"], st["Qinv"], st["Rinv"], dev["A"], dev["Bu"],
                       dev["q"], dev["r"], 1e-6, 2000, st["lam"], st["dz"], st["iters"], st["relres"], st["flags"])
    torch.cuda.synchronize()
    o_form = oracle.form_schur(*synth.inputs(bt))
    o = oracle.pcg_solve(o_form["S"], o_form["Pinv"], o_form["gamma"], o_form["Qinv"], o_form["Rinv"], bt["A"],
                         bt["Bu"], bt["q"], bt["r"], 1e-6, 2000)
    it, fl = st["iters"].cpu().numpy(), st["flags"].cpu().numpy()
    ratio = it / np.maximum(o["iters"], 1)
    err = rel_rows(st["dz"].cpu().numpy(), o["dz"])
    print("iters gpu %d..%d (median %.0f), oracle %d..%d (median %.0f); ratio %.3f..%.3f median %.3f; "
          "dz rel err max %.3e" % (it.min(), it.max(), np.median(it), o["iters"].min(), o["iters"].max(),
                                   np.median(o["iters"]), ratio.min(), ratio.max(), np.median(ratio), err.max()))
    assert (fl == 0).all() and (o["flags"] == 0).all()
    assert (it < 2000).all()
    assert ratio.min() >= 0.75 and ratio.max() <= 1.5
    assert 0.9 <= np.median(ratio) <= 1.15
    assert err.max() <= 1e-3


def test_pcg_respects_the_iteration_cap_where_the_preconditioner_turns_indefinite():
    """Within one workgroup's horizon (N = 64, register-resident rows) on the
    ill-conditioned workload's generators, the assembled fp32 Phi^-1 is not positive
    definite on some solves.  A solve whose r'z stops being positive switches to the
    factored form with the iterations left: iters never exceeds max_iters, a solve at the
    cap is flagged, and every solve not flagged meets the exit test, with a true residual
    (fp64, on the oracle's S) within 5e-5.  (With cond(S) ~ 1e6 a residual of 1e-6
    bounds dz only loosely: on this batch one converged solve sits 3.3e-3 from the
    oracle's PCG step, the others within 6e-4.  These horizons are off the workload
    list; the ill-conditioned workload itself runs at N = 128.)"""
    bt = _batch(5, 512, N=64)
    dims = bt["dims"]
    _ident("pcg cap, workload 5 generators at N = 64", dims)
    o_form = oracle.form_schur(*synth.inputs(bt))
    o = oracle.pcg_solve(o_form["S"], o_form["Pinv"], o_form["gamma"], o_form["Qinv"], o_form["Rinv"], bt["A"],
                         bt["Bu"], bt["q"], bt["r"], 1e-6, 2000)
    for cap in (2000, 300):
        dev = ops.to_device(bt)
        st = ops.alloc_outputs(dims, 8)
        ops.gato_form_schur(dims, *[dev[f] for f in synth.FIELDS], None, st["S"], st["Pinv"], st["gamma"],
                            st["Qinv"], st["Rinv"], st["flags"])
        st["lam"].zero_()
        st["flags"].zero_()
        ops.gato_pcg_solve(dims, st["S"], st["Pinv"], st["gamma"], st["Qinv"], st["Rinv"], dev["A"], dev["Bu"],
                           dev["q"], dev["r"], 1e-6, cap, st["lam"], st["dz"], st["iters"], st["relres"], st["flags"])
        torch.cuda.synchronize()
        it, fl, rr = st["iters"].cpu().numpy(), st["flags"].cpu().numpy(), st["relres"].cpu().numpy()
        capped = (fl & ops.F_PCG_MAXITER) != 0
        done = ~capped
        err = rel_rows(st["dz"].cpu().numpy(), o["dz"])
        true_res = btd_relres(o_form["S"], o_form["gamma"], st["lam"].cpu().numpy())
        print("cap %d: iters max %d, capped %d, oracle iters max %d; not capped: true residual max %.2e, "
              "dz err vs the oracle's PCG step max %.3e, over 1e-3 %d" % (
                  cap, it.max(), capped.sum(), o["iters"].max(), true_res[done].max(initial=0.0),
                  err[done].max(initial=0.0), (err[done] > 1e-3).sum()))
        assert (it <= cap).all()
        assert (it[capped] == cap).all()
        assert (fl & ~ops.F_PCG_MAXITER == 0).all()
        assert (rr[done] <= 1e-6).all()
        assert (true_res[done] <= 5e-5).all()
        if cap < o["iters"].min():
            assert capped.all()


def test_pcg_warm_start_and_flags():
    bt = _batch(3, 4)
    o_form = oracle.form_schur(*synth.inputs(bt))
    exact = oracle.direct_solve(o_form["S"], o_form["gamma"])["lam"]
    warm = gpu_pcg(bt, o_form, 1e-6, 200, lambda0=exact)
    assert (warm["iters"] <= 1).all()
    # the cap is honoured: one iteration, then the flag
    capped = gpu_pcg(bt, o_form, 1e-6, 1)
    assert (capped["flags"] & ops.F_PCG_MAXITER).all() and (capped["iters"] == 1).all()
    bad = dict(o_form)
    bad["gamma"] = o_form["gamma"].copy()
    bad["gamma"][2, 3, 1] = np.nan
    res = gpu_pcg(bt, bad, 1e-6, 200, flags=np.array([0, 32, 0, 0]))
    assert res["flags"][2] & ops.F_NONFINITE
    assert res["flags"][1] == 32  # ORed into existing bits
    z = dict(o_form)
    z["gamma"] = np.zeros_like(o_form["gamma"])
    zr = gpu_pcg(bt, z, 1e-6, 200, lambda0=np.ones_like(exact))
    assert (zr["iters"] == 0).all() and np.all(zr["lam"] == 0) and (zr["relres"] == 0).all()


# ---------------------------------------------------------------- stage 3


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_merit_parity(cid):
    B = SMALL[cid]
    _ident("merit", cid, B)
    bt = _batch(cid, B)
    ref_step = oracle.sqp_step(*synth.inputs(bt), None, 1e-6, CAPS[cid], A64, 1.0)
    dz32 = ref_step["dz"].astype(np.float32)
    for mu in (1.0, 7.5):
        g = gpu_merit(bt, dz32, mu)
        o = oracle.merit_eval(*synth.inputs(bt), dz32.astype(np.float64), A64, mu)
        assert merit_rel(g["merit"], o).max() <= 1e-4
        assert (np.abs(g["merit0"] - o["merit0"]) <= 1e-4 * o["merit0"]).all()
        np.testing.assert_array_equal(g["best"], select(g["merit"], g["merit0"]))
        np.testing.assert_array_equal(g["flags"] & ops.F_LS_FAILED, np.where(g["best"] < 0, ops.F_LS_FAILED, 0))


def test_merit_bit_identical_across_workgroup_sizes():
    """The bit-identity gate: every launch variant of the merit (workgroup size, and the
    fused per-knot or candidate-parallel decomposition) gives the same bits."""
    bt = _batch(5, 3)
    dz = np.random.default_rng(0).standard_normal((3, 128 * 14 + 127 * 7)).astype(np.float32) * 0.1
    runs = [gpu_merit(bt, dz, 1.3, flags=np.array([0, 64, 0], np.int32))]  # gato_merit_eval's own choice
    for variant in (ops.MERIT_PER_KNOT, ops.MERIT_PER_CANDIDATE):
        for w in (0, 1, 2, 3, 8, 16):
            runs.append(gpu_merit(bt, dz, 1.3, flags=np.array([0, 64, 0], np.int32), variant=variant, waves=w))
    for r in runs[1:]:
        for k in ("merit", "merit0", "best", "flags"):
            np.testing.assert_array_equal(r[k], runs[0][k])
    assert runs[0]["flags"][1] & 64  # ORed into the bits already there


@pytest.mark.parametrize("cid,B,N", [(3, 4, 300), (3, 64, 128), (5, 8, 100), (4, 2, 1024)])
def test_step_merit_split_is_bit_identical(cid, B, N):
    """On horizons beyond the fused path, gato_sqp_step spreads a solve's merit knots
    over several workgroups when the batch is small; its sums must carry the same bits
    as gato_merit_eval's one-workgroup-per-solve kernel on the same dz."""
    _ident("merit split", cid, B, N)
    bt = _batch(cid, B, N=N)
    g = gpu_sqp(bt, 1e-6, CAPS[cid])
    m = gpu_merit(bt, g["dz"], 1.0)
    for k in ("merit", "merit0", "best"):
        np.testing.assert_array_equal(g[k], m[k])
    np.testing.assert_array_equal(g["flags"] & ops.F_LS_FAILED, m["flags"] & ops.F_LS_FAILED)


def test_merit_ascent_direction_fails_line_search():
    bt = _batch(2, 2)
    bt["x0"][:] = 0
    bt["e"][:] = 0
    ref = oracle.sqp_step(*synth.inputs(bt), None, 1e-8, 400, A64, 1.0)
    g = gpu_merit(bt, -ref["dz"].astype(np.float32), 1.0)
    assert (g["best"] == -1).all() and (g["flags"] & ops.F_LS_FAILED).all()


# ---------------------------------------------------------------- whole step


SQP_CASES = [(1, 1), (2, 1), (2, 8), (2, 16), (3, 1), (3, 8), (3, 16), (3, 64), (3, 128), (4, 16), (4, 64), (4, 256),
             (5, 512)]


@pytest.mark.parametrize("cid,B", SQP_CASES, ids=["cfg%d-B%d" % c for c in SQP_CASES])
def test_sqp_step_parity(cid, B):
    """gato_sqp_step as shipped, every solve of every batch against the oracle."""
    _ident("sqp_step", cid, B)
    bt = _batch(cid, B)
    g = gpu_sqp(bt, 1e-6, CAPS[cid])
    ins = synth.inputs(bt)
    if _direct_path(bt):
        # the step comes from the direct solve and its refinement pass: compare with the
        # oracle's exact step (block Cholesky of S) and the stage-1 flag bits
        f = oracle.form_schur(*ins)
        lam = oracle.direct_solve(f["S"], f["gamma"])["lam"]
        o = {"dz": oracle.recover(f["Qinv"], f["Rinv"], bt["A"], bt["Bu"], bt["q"], bt["r"], lam),
             "flags": f["flags"]}
        assert (g["iters"] == 0).all()
    else:
        o = oracle.sqp_step(*ins, None, 1e-6, CAPS[cid], A64, 1.0)
    err = rel_rows(g["dz"], o["dz"])
    print("cfg%d B%d: dz rel err max %.3e median %.3e; iters gpu %d..%d" % (
        cid, B, err.max(), np.median(err), g["iters"].min(), g["iters"].max()))
    assert err.max() <= 1e-3
    assert ((g["flags"] & ~ops.F_LS_FAILED) == (o["flags"] & ~ops.F_LS_FAILED)).all()
    # merit of the GPU's own step, against the oracle's merit of that same step
    om = oracle.merit_eval(*ins, g["dz"].astype(np.float64), A64, 1.0)
    assert merit_rel(g["merit"], om).max() <= 1e-4
    np.testing.assert_array_equal(g["best"], select(g["merit"], g["merit0"]))
    if _direct_path(bt):
        # and the merits of the oracle's exact step: the step is exact within the bars
        oe = oracle.merit_eval(*ins, o["dz"], A64, 1.0)
        me = merit_rel(g["merit"], oe)
        print("merit vs the exact step's: max %.3e" % me.max())
        assert me.max() <= 1e-4
        np.testing.assert_array_equal(g["best"], oe["best"])
    else:
        assert np.abs(g["iters"] - o["iters"]).max() <= 2


def test_fused_step_equals_staged_calls():
    """gato_sqp_step (one fused kernel) and form -> pcg -> merit give identical bits."""
    bt = _batch(3, 16)
    fused = gpu_sqp(bt, 1e-6, 200)
    f = gpu_form(bt)
    p = gpu_pcg(bt, f, 1e-6, 200)
    m = gpu_merit(bt, p["dz"], 1.0)
    np.testing.assert_array_equal(fused["dz"], p["dz"])
    np.testing.assert_array_equal(fused["lam"], p["lam"])
    np.testing.assert_array_equal(fused["iters"], p["iters"])
    np.testing.assert_array_equal(fused["merit"], m["merit"])
    np.testing.assert_array_equal(fused["merit0"], m["merit0"])
    np.testing.assert_array_equal(fused["best"], m["best"])


def test_fused_step_equals_staged_calls_through_breakdowns():
    """Indefinite problems (Q_k = -I at one knot, of several sizes), where PCG stops at
    p'Sp <= 0 or r'z <= 0: the fused kernel, which takes the residual's step before it
    knows of a breakdown and restores r'r at the exit, gives the bits of the staged
    calls, which keep r as it was; at least one solve ends in a breakdown."""
    bt = _batch(3, 16)
    for b in range(16):
        bt["Q"][b, 4 + 3 * b] = (-0.05 * (b + 1)) * np.eye(14, dtype=np.float32)
    fused = gpu_sqp(bt, 1e-6, 200)
    f = gpu_form(bt)
    p = gpu_pcg(bt, f, 1e-6, 200)
    print("flags", fused["flags"].tolist(), "iters", fused["iters"].tolist())
    assert (fused["flags"] & ops.F_PCG_BREAKDOWN).any()
    for key in ("lam", "dz", "iters", "relres"):
        np.testing.assert_array_equal(fused[key], p[key], err_msg=key)
    np.testing.assert_array_equal(fused["flags"] & ~ops.F_LS_FAILED, (f["flags"] | p["flags"]) & ~ops.F_LS_FAILED)


def test_solve_independent_of_batch_position():
    big = _batch(2, 16)
    g = gpu_sqp(big, 1e-6, 200)
    for b in (0, 7, 15):
        one = _batch(2, 1, first=b)
        h = gpu_sqp(one, 1e-6, 200)
        np.testing.assert_array_equal(h["dz"][0], g["dz"][b])
        np.testing.assert_array_equal(h["merit"][0], g["merit"][b])


@pytest.mark.parametrize("cid,B", [(3, 16384), (5, 4096)])
def test_large_batches_give_every_copy_the_same_bits(cid, B):
    """Batches far beyond one round of workgroups (16384 fused steps; 4096 long-horizon steps
    through the direct solve and its refinement pass): 32 generated solves tiled B/32 times.
    Every copy must give the bits of the first, and the first copies meet the oracle's bars."""
    _ident("large batch", cid, B)
    T = 32
    base = _batch(cid, T)
    big = {f: np.tile(base[f], (B // T,) + (1,) * (base[f].ndim - 1)) for f in synth.FIELDS}
    n, m, N, _ = base["dims"]
    big["dims"] = (n, m, N, B)
    g = gpu_sqp(big, 1e-6, CAPS[cid])
    del big
    for key in ("lam", "dz", "merit", "merit0", "best", "iters", "relres", "flags"):
        a = g[key].reshape((B // T, T) + g[key].shape[1:])
        assert np.array_equal(a, np.broadcast_to(a[:1], a.shape)), key
    first = {k: g[k][:T] for k in ("dz", "merit", "merit0", "best", "iters", "flags")}
    ins = synth.inputs(base)
    if _direct_path(base):
        f = oracle.form_schur(*ins)
        lam = oracle.direct_solve(f["S"], f["gamma"])["lam"]
        o = {"dz": oracle.recover(f["Qinv"], f["Rinv"], base["A"], base["Bu"], base["q"], base["r"], lam),
             "flags": f["flags"]}
        assert (first["iters"] == 0).all()
    else:
        o = oracle.sqp_step(*ins, None, 1e-6, CAPS[cid], A64, 1.0)
        assert np.abs(first["iters"] - o["iters"]).max() <= 2
    assert rel_rows(first["dz"], o["dz"]).max() <= 1e-3
    assert ((first["flags"] & ~ops.F_LS_FAILED) == (o["flags"] & ~ops.F_LS_FAILED)).all()
    om = oracle.merit_eval(*ins, first["dz"].astype(np.float64), A64, 1.0)
    assert merit_rel(first["merit"], om).max() <= 1e-4
    np.testing.assert_array_equal(first["best"], select(first["merit"], first["merit0"]))


def test_stage_times_reported():
    g = gpu_sqp(_batch(3, 8), 1e-6, 200, times=True)
    assert g["times"].total_us > 0
    g5 = gpu_sqp(_batch(5, 2), 1e-6, 2000, times=True)
    assert g5["times"].schur_us > 0 and g5["times"].linsys_us > 0 and g5["times"].merit_us > 0


# ---------------------------------------------------------------- edge cases


@pytest.mark.parametrize("N", [1, 2, 5, 37, 63, 64, 65, 100, 128, 129, 200, 256])
def test_ragged_and_extreme_horizons(N):
    """Horizons that leave a wave partly empty, fill a workgroup exactly, or spill into the
    long-horizon path (windowed formation, direct block-tridiagonal solve)."""
    _ident("horizon", N)
    bt = _batch(3, 3, N=N)
    g = gpu_sqp(bt, 1e-6, 400, rho=np.array([0.0, 0.1, 1.0]))
    o = oracle.sqp_step(*synth.inputs(bt), np.array([0.0, 0.1, 1.0]), 1e-6, 400, A64, 1.0)
    assert rel_rows(g["dz"], o["dz"]).max() <= 1e-3
    if _direct_path(bt):
        assert (g["iters"] == 0).all() and (g["flags"] & ~ops.F_LS_FAILED == 0).all()
    om = oracle.merit_eval(*synth.inputs(bt), g["dz"].astype(np.float64), A64, 1.0)
    assert merit_rel(g["merit"], om).max() <= 1e-4
    f = gpu_form(bt, rho=np.array([0.0, 0.1, 1.0]))
    of = oracle.form_schur(*synth.inputs(bt), rho=np.array([0.0, 0.1, 1.0]))
    assert rel_rows(f["S"], of["S"]).max() <= 1e-5 and rel_rows(f["Pinv"], of["Pinv"]).max() <= 1e-4


@pytest.mark.parametrize("cid,N", [(1, 1), (4, 1), (4, 3), (4, 17), (4, 32), (2, 65)])
def test_other_shapes_edges(cid, N):
    bt = _batch(cid, 2, N=N)
    g = gpu_sqp(bt, 1e-6, 400)
    o = oracle.sqp_step(*synth.inputs(bt), None, 1e-6, 400, A64, 1.0)
    assert rel_rows(g["dz"], o["dz"]).max() <= 1e-3


def test_zero_batch_is_a_no_op():
    bt = _batch(3, 1)
    n, m, N, _ = bt["dims"]
    empty = {f: bt[f][:0] for f in synth.FIELDS}
    empty["dims"] = (n, m, N, 0)
    r = gpu_sqp(empty, 1e-6, 200)
    assert r["dz"].shape == (0, N * n + (N - 1) * m)


def test_golden_examples_on_gpu():
    import json

    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "scalar_lq.json")))["cases"]
    for c in cases:
        bt = {k: np.asarray(c[k], np.float32)[None] for k in synth.FIELDS}
        bt["dims"] = (1, 1, 2, 1)
        al = np.array([float(a) for a in c["merit_at"]], np.float32)
        g = gpu_sqp(bt, 1e-6, 10, mu=c["mu"], alphas=al)
        np.testing.assert_allclose(g["dz"][0], c["dz"], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(g["lam"][0], c["lambda"], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(g["merit"][0], list(c["merit_at"].values()), rtol=1e-5, atol=1e-6)
        assert g["iters"][0] == c["pcg_iters"] and g["best"][0] == c["best"]
        f = gpu_form(bt)
        np.testing.assert_allclose(f["S"][0], c["S"], rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(f["Pinv"][0], c["Pinv"], rtol=1e-6, atol=1e-7)


def test_step_flags_match_oracle():
    bt = _batch(3, 4)
    bt["e"][1, 10, 3] = np.nan
    bt["Q"][2, 20] = -np.eye(14, dtype=np.float32)
    g = gpu_sqp(bt, 1e-6, 200)
    o = oracle.sqp_step(*synth.inputs(bt), None, 1e-6, 200, A64, 1.0)
    for b in (0, 3):
        assert (g["flags"][b] & ~ops.F_LS_FAILED) == (o["flags"][b] & ~ops.F_LS_FAILED) == 0
    assert g["flags"][1] & ops.F_NONFINITE and o["flags"][1] & ops.F_NONFINITE
    assert g["flags"][2] & ops.F_Q_NOT_SPD and o["flags"][2] & ops.F_Q_NOT_SPD
