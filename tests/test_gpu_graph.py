"""gato_sqp_step captured in a HIP graph and replayed (the use the allocation-free entry
point is for): every replay gives the bits of the eager call, on the fused path, the
long-horizon paths (resident reduction with its in-kernel refinement pass; nested
dissection with the separate refinement kernels) and a padded shape, with the caller's
workspace and with the library's fixed scratch. Between replays the outputs are
overwritten and the same step runs eagerly on other inputs, so a replay that left an
output unwritten or read a stale one would show."""
import numpy as np
import pytest
import torch

from block_tridiagonal_pcg_amd import ops, synth

pytestmark = pytest.mark.gpu

FIELDS = ("lam", "dz", "merit", "merit0", "best", "iters", "relres", "flags")
CAPS = {1: 200, 2: 200, 3: 200, 4: 200, 5: 2000}

# (generators of workload, B, n, m, N, allocation-free)
CASES = [
    (3, 16, 14, 7, 64, False),   # fused, no workspace
    (3, 16, 14, 7, 64, True),
    (5, 16, 14, 7, 128, False),  # resident cyclic reduction with its in-kernel refinement pass
    (5, 16, 14, 7, 128, True),
    (3, 4, 14, 7, 300, True),    # nested dissection, refinement kernels
    (2, 8, 10, 5, 32, False),    # padded into (12, 6): copy kernels around the fused step
    (4, 8, 24, 12, 16, True),    # 32-lane groups, fused
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.load()


def _step(bt, noalloc):
    """A closure that runs the step on bt's device copy into its own outputs."""
    dims = bt["dims"]
    dev = ops.to_device(bt)
    out = ops.alloc_outputs(dims, 8)
    ws = None if noalloc else ops.workspace_for(dims, 8)
    cid = bt["cid"]
    args = [dev[f] for f in synth.FIELDS] + [None, 1e-6, CAPS[cid], synth.ALPHAS, 1.0] + [out[k] for k in FIELDS]

    def run():
        if noalloc:
            ops.gato_sqp_step_noalloc(dims, *args)
        else:
            ops.gato_sqp_step(dims, *args, workspace=ws)

    return run, out


def _reset(out):
    """Cold start (lambda is the step's input) and garbage in every other output."""
    out["lam"].zero_()
    for k in ("dz", "merit", "merit0", "relres"):
        out[k].fill_(float("nan"))
    for k in ("best", "iters", "flags"):
        out[k].fill_(-7)


def _host(out):
    return {k: out[k].cpu().numpy().copy() for k in FIELDS}


@pytest.mark.parametrize("case", CASES, ids=["c%d-B%d-n%dm%dN%d-%s" % (c[:5] + ("noalloc" if c[5] else "ws",))
                                             for c in CASES])
def test_step_replayed_from_a_graph_matches_the_eager_call(case):
    cid, B, n, m, N, noalloc = case
    print("case: graph", case, flush=True)
    bt = synth.make_batch(cid, B, n=n, m=m, N=N)
    bt["cid"] = cid
    other = synth.make_batch(cid, B, n=n, m=m, N=N, first=B)
    other["cid"] = cid
    run, out = _step(bt, noalloc)
    run_o, out_o = _step(other, noalloc)

    _reset(out)
    run()
    torch.cuda.synchronize()
    ref = _host(out)
    _reset(out_o)
    run_o()
    torch.cuda.synchronize()
    ref_o = _host(out_o)
    assert not np.isnan(ref["dz"]).any() and (ref["iters"] >= 0).all()

    g = torch.cuda.CUDAGraph()
    _reset(out)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        _reset(out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _host(out)
        for k in FIELDS:
            np.testing.assert_array_equal(got[k], ref[k], err_msg="replay %d, %s" % (rep, k))
        # eager work between replays: the same step on other inputs (sharing the scratch
        # array when allocation-free), checked against its own eager result
        _reset(out_o)
        run_o()
        torch.cuda.synchronize()
        got_o = _host(out_o)
        for k in FIELDS:
            np.testing.assert_array_equal(got_o[k], ref_o[k], err_msg="eager call after replay %d, %s" % (rep, k))
