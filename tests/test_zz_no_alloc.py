"""gato_sqp_step_noalloc (the entry point for callers that cannot allocate) against
gato_sqp_step with a caller-owned workspace, through the C ABI: identical bits on two
calls in a row, the second with a smaller problem, plus the fused path (no scratch)
and the size limit."""
import numpy as np
import pytest
import torch

from block_tridiagonal_pcg_amd import ops, synth

pytestmark = pytest.mark.gpu

FIELDS = ("lam", "dz", "merit", "merit0", "best", "iters", "relres", "flags")


def _run(bt, noalloc, cap=200):
    dims = bt["dims"]
    dev = ops.to_device(bt)
    out = ops.alloc_outputs(dims, 8)
    for k in ("lam", "dz", "merit", "merit0", "relres"):
        out[k].fill_(float("nan"))
    args = [dev[f] for f in synth.FIELDS] + [None, 1e-6, cap, synth.ALPHAS, 1.0] + [out[k] for k in FIELDS]
    if noalloc:
        ops.gato_sqp_step_noalloc(dims, *args)
    else:
        ws = ops.workspace_for(dims, 8)
        if ws is not None:
            ws.fill_(255)
        ops.gato_sqp_step(dims, *args, workspace=ws)
    torch.cuda.synchronize()
    return {k: out[k].cpu().numpy() for k in FIELDS}


@pytest.mark.parametrize("first,second", [((3, 16, 128), (3, 4, 100)), ((5, 24, 128), (4, 3, 40)),
                                          ((3, 8, 300), (3, 2, 65))])
def test_noalloc_equals_the_workspace_call(first, second):
    for cid, B, N in (first, second):
        print("case: noalloc", cid, B, N, flush=True)
        bt = synth.make_batch(cid, B, N=N)
        assert ops.gato_workspace_bytes(bt["dims"]) <= ops.NOALLOC_SCRATCH_BYTES
        ref = _run(bt, False, 2000 if cid == 5 else 200)
        got = _run(bt, True, 2000 if cid == 5 else 200)
        for k in FIELDS:
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        assert (got["flags"] & ~ops.F_LS_FAILED == 0).all()


def test_noalloc_fused_path_and_limit():
    bt = synth.make_batch(3, 8)  # N = 64: fused, no scratch
    ref, got = _run(bt, False), _run(bt, True)
    for k in FIELDS:
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    big = (14, 7, 128, 512)
    assert ops.gato_workspace_bytes(big) > ops.NOALLOC_SCRATCH_BYTES
    al = (ops.ctypes.c_float * 8)(*synth.ALPHAS)
    # the host rejects the dims before looking at any pointer or touching the device
    rc = ops.load().gato_sqp_step_noalloc(ops.ctypes.byref(ops.Dims(*big)), *[None] * 9, 1e-6, 200, al, 8, 1.0,
                                          *[None] * 8, None)
    assert rc == ops.E_WORKSPACE
