"""Host-side logic of bench.py (no GPU): the algorithmic byte counts it prices the
roofline with, pinned against the arrays the workloads actually hold; the source
digest that gates the committed traffic figure; and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from block_tridiagonal_pcg_amd import ops, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_input_bytes_equal_the_generated_arrays(cid):
    bt = synth.make_batch(cid, 1)
    n, m, N, _ = bt["dims"]
    held = sum(np.asarray(bt[f], np.float32).nbytes for f in synth.FIELDS)
    assert bench.input_bytes(n, m, N) == held


@pytest.mark.parametrize("n,m,N,na", [(14, 7, 64, 8), (4, 2, 8, 3), (24, 12, 16, 16), (1, 1, 1, 1)])
def test_output_bytes_equal_the_step_outputs(n, m, N, na):
    sh = ops._shapes(n, m, N, 1)
    per_solve = np.prod(sh["lam"]) + np.prod(sh["dz"]) + na + 5  # merit[n_alpha]; merit0, best, iters, relres, flags
    assert bench.output_bytes(n, m, N, na) == 4 * per_solve


@pytest.mark.parametrize("n,N", [(1, 1), (2, 3), (3, 5), (14, 4)])
def test_pcg_bytes_count_the_unique_entries_of_s_and_phi(n, N):
    """Unique entries of a symmetric block-tridiagonal matrix (the upper triangle of its
    dense pattern), for S and Phi^-1, in fp32."""
    K = N * n
    pat = np.zeros((K, K), bool)
    for k in range(N):
        for j in (k - 1, k, k + 1):
            if 0 <= j < N:
                pat[k * n:(k + 1) * n, j * n:(j + 1) * n] = True
    assert bench.pcg_iter_bytes(n, N) == 4 * 2 * int(np.triu(pat).sum())


def test_source_digest_ignores_comments_only():
    files = {f: open(os.path.join(ROOT, f)).read() for f in bench.FUSED_SOURCES}
    base = bench.source_digest(read=files.__getitem__)
    assert base == bench.source_digest()
    f0 = bench.FUSED_SOURCES[0]
    commented = dict(files)
    commented[f0] = "// a comment\n/* and a\n   block comment */\n" + files[f0].replace("\n", "  \n", 3)
    assert bench.source_digest(read=commented.__getitem__) == base
    changed = dict(files)
    changed[f0] = files[f0] + "\nstatic int extra_symbol;\n"
    assert bench.source_digest(read=changed.__getitem__) != base


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_rel_err_rows():
    o = np.array([[3.0, 4.0], [1.0, 0.0]])
    g = np.array([[3.0, 4.5], [1.0, 0.0]])
    np.testing.assert_allclose(bench.rel_err_rows(g, o), [0.1, 0.0])


def test_exact_step_matches_the_oracle_step():
    """The direct-solve reference bench.py reports against: on a well-conditioned batch
    it equals the oracle's PCG step to within PCG's tolerance."""
    import oracle

    bt = synth.make_batch(1, 3)
    ex = bench.exact_step(bt, 8)
    al = np.array([2.0 ** -i for i in range(8)])
    st = oracle.sqp_step(*[bt[f] for f in ("Q", "q", "R", "r", "A", "Bu", "e", "x0")], None, 1e-10, 500, al,
                         bench.MU)
    assert bench.rel_err_rows(ex["dz"], st["dz"]).max() < 1e-7
    assert bench.rel_err_rows(ex["merit"].reshape(-1, 1), st["merit"].reshape(-1, 1)).max() < 1e-7
    assert (ex["best"] == st["best"]).all()


def test_cpu_baseline_reports_all_cores_one_core_and_stages():
    """The CPU-baseline leg's record: all-thread and one-thread rates, the oracle's
    stages, CPU model and compiler, and the oracle's step as its second value."""
    import oracle

    bt = synth.make_batch(2, 4)
    bt["cid"] = 2
    rec, first = bench.cpu_baseline(bt, 8, 0.5)
    assert rec["kind"] == "oracle" and rec["unit"] == "solves/s" and rec["value"] > 0
    assert rec["cores"] == oracle.num_threads()
    assert rec["one_core"]["cores"] == 1 and rec["one_core"]["value"] > 0
    assert all(rec["stage_us"][k] > 0 for k in ("schur_us", "linsys_us", "merit_us"))
    assert rec["compiler"].startswith("gcc ") and "-fno-fast-math" in rec["compiler"]
    assert rec["cpu_model"]
    assert oracle.num_threads() == rec["cores"]  # the thread count is restored
    assert first["dz"].shape == (4, 32 * 12 + 31 * 6)
