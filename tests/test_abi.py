"""Boundary checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before enqueuing anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _headers():
    inc = os.path.join(ROOT, "include")
    return "\n".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))


def _declared():
    text = _headers()
    return sorted(set(re.findall(r"^\s*(?:int32_t|int|size_t|const char\*)\s+(gato_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    from block_tridiagonal_pcg_amd import ops

    if not os.path.exists(ops.library_path()):
        pytest.fail("libgato.so is not built; run __graft_entry__.build()")
    return ops.load()


def _prototypes():
    """{function: [(type, name), ...]} of every declaration in the header."""
    text = re.sub(r"/\*.*?\*/", " ", _headers(), flags=re.S)
    out = {}
    for m in re.finditer(r"(?:int32_t|int|size_t|const char\*)\s+(gato_\w+)\s*\(([^)]*)\)\s*;", text):
        params = []
        for arg in m.group(2).split(","):
            arg = " ".join(arg.split())
            if arg in ("", "void"):
                continue
            name = re.search(r"(\w+)$", arg).group(1)
            params.append((arg[: -len(name)].replace(" *", "*").strip(), name))
        out[m.group(1)] = params
    return out


# The four calls of the boundary, argument by argument (type, name), as the QP data
# enters them: the problem arrays in the order the paper states the problem, then the
# stage's outputs, then the stream.
BOUNDARY = {
    "gato_form_schur": [
        ("const gato_dims_t*", "dims"), ("const float*", "Q"), ("const float*", "q"), ("const float*", "R"),
        ("const float*", "r"), ("const float*", "A"), ("const float*", "Bu"), ("const float*", "e"),
        ("const float*", "x0"), ("const float*", "rho"), ("float*", "S"), ("float*", "Pinv"), ("float*", "gamma"),
        ("float*", "Qinv"), ("float*", "Rinv"), ("int32_t*", "flags"), ("hipStream_t", "stream")],
    "gato_pcg_solve": [
        ("const gato_dims_t*", "dims"), ("const float*", "S"), ("const float*", "Pinv"), ("const float*", "gamma"),
        ("const float*", "Qinv"), ("const float*", "Rinv"), ("const float*", "A"), ("const float*", "Bu"),
        ("const float*", "q"), ("const float*", "r"), ("float", "eps"), ("int32_t", "max_iters"),
        ("float*", "lambda"), ("float*", "dz"), ("int32_t*", "iters"), ("float*", "relres"), ("int32_t*", "flags"),
        ("hipStream_t", "stream")],
    "gato_merit_eval": [
        ("const gato_dims_t*", "dims"), ("const float*", "Q"), ("const float*", "q"), ("const float*", "R"),
        ("const float*", "r"), ("const float*", "A"), ("const float*", "Bu"), ("const float*", "e"),
        ("const float*", "x0"), ("const float*", "dz"), ("const float*", "alphas_host"), ("int32_t", "n_alpha"),
        ("float", "mu"), ("float*", "merit"), ("float*", "merit0"), ("int32_t*", "best"), ("int32_t*", "flags"),
        ("hipStream_t", "stream")],
    "gato_sqp_step": [
        ("const gato_dims_t*", "dims"), ("const float*", "Q"), ("const float*", "q"), ("const float*", "R"),
        ("const float*", "r"), ("const float*", "A"), ("const float*", "Bu"), ("const float*", "e"),
        ("const float*", "x0"), ("const float*", "rho"), ("float", "eps"), ("int32_t", "max_iters"),
        ("const float*", "alphas_host"), ("int32_t", "n_alpha"), ("float", "mu"), ("float*", "lambda"),
        ("float*", "dz"), ("float*", "merit"), ("float*", "merit0"), ("int32_t*", "best"), ("int32_t*", "iters"),
        ("float*", "relres"), ("int32_t*", "flags"), ("void*", "workspace"), ("size_t", "workspace_bytes"),
        ("gato_stage_times_t*", "times"), ("hipStream_t", "stream")],
    "gato_workspace_bytes": [("const gato_dims_t*", "dims"), ("int32_t", "n_alpha")],
    "gato_status_string": [("int", "code")],
}


def test_header_declares_the_abi():
    assert _declared() == sorted([
        "gato_cr_levels", "gato_cr_solve", "gato_cr_workspace_bytes",
        "gato_direct_solve", "gato_direct_workspace_bytes", "gato_form_schur", "gato_merit_eval",
        "gato_merit_eval_shape", "gato_pcg_solve", "gato_shape_supported", "gato_sqp_step",
        "gato_sqp_step_noalloc", "gato_sqp_step_opts", "gato_status_string", "gato_step_solver",
        "gato_workspace_bytes", "gato_step_workspace_bytes", "gato_chain_qp", "gato_take_step"])


def test_driver_calls_validate_on_the_host(lib):
    """The SQP driver's kernels: bad dims and parameters return before any launch."""
    from block_tridiagonal_pcg_amd import ops, synth

    prm = ops.chain_params(synth.Chain(7))
    P = [ctypes.c_void_p(4096 * (j + 1)) for j in range(12)]
    f = lib.gato_chain_qp
    assert f(ctypes.byref(ops.Dims(14, 7, 16, 2)), None, *P, None) == ops.E_NULL
    assert f(ctypes.byref(ops.Dims(12, 7, 16, 2)), ctypes.byref(prm), *P, None) == ops.E_DIMS  # n != 2 dof
    assert f(ctypes.byref(ops.Dims(14, 6, 16, 2)), ctypes.byref(prm), *P, None) == ops.E_DIMS  # m != dof
    assert f(ctypes.byref(ops.Dims(14, 7, 1, 2)), ctypes.byref(prm), *P, None) == ops.E_DIMS   # no dynamics
    assert f(ctypes.byref(ops.Dims(14, 7, 16, 2)), ctypes.byref(prm), *P[:11], None, None) == ops.E_NULL
    assert f(ctypes.byref(ops.Dims(14, 7, 16, 0)), ctypes.byref(prm), *[None] * 12, None) == ops.OK
    bad = ops.chain_params(synth.Chain(7, h=0.0))
    assert f(ctypes.byref(ops.Dims(14, 7, 16, 2)), ctypes.byref(bad), *P, None) == ops.E_PARAM
    g = lib.gato_take_step
    al = (ctypes.c_float * 8)(*[2.0 ** -i for i in range(8)])
    d = ctypes.byref(ops.Dims(14, 7, 16, 2))
    assert g(d, al, 0, *P[:5], 1e-8, 10.0, None) == ops.E_PARAM
    assert g(d, al, 17, *P[:5], 1e-8, 10.0, None) == ops.E_PARAM
    assert g(d, al, 8, *P[:5], 0.0, 10.0, None) == ops.E_PARAM
    assert g(d, al, 8, *P[:5], 1.0, 0.5, None) == ops.E_PARAM
    assert g(d, None, 8, *P[:5], 1e-8, 10.0, None) == ops.E_NULL
    assert g(d, al, 8, None, *P[1:5], 1e-8, 10.0, None) == ops.E_NULL
    assert g(ctypes.byref(ops.Dims(14, 7, 16, 0)), al, 8, *[None] * 5, 1e-8, 10.0, None) == ops.OK


def test_boundary_signatures():
    """The header's argument lists of the boundary calls, type and name, in order."""
    protos = _prototypes()
    for fn, args in BOUNDARY.items():
        assert protos[fn] == args, fn
    # the variants add their choices just before the stream and change nothing else
    assert protos["gato_sqp_step_opts"] == BOUNDARY["gato_sqp_step"][:-1] + [
        ("const gato_step_opts_t*", "opts"), ("hipStream_t", "stream")]
    assert protos["gato_merit_eval_shape"] == BOUNDARY["gato_merit_eval"][:-1] + [
        ("int32_t", "variant"), ("int32_t", "waves"), ("hipStream_t", "stream")]
    # the allocation-free step: no workspace and no stage times (nothing that allocates)
    assert protos["gato_sqp_step_noalloc"] == BOUNDARY["gato_sqp_step"][:-4] + [("hipStream_t", "stream")]


def test_noalloc_rejects_dims_beyond_its_scratch(lib):
    """The allocation-free step serves the fused horizons without scratch and longer
    ones within its fixed array; beyond it the host returns E_WORKSPACE before looking
    at any pointer or touching a device (none is present here)."""
    from block_tridiagonal_pcg_amd import ops

    text = open(os.path.join(ROOT, "include", "gato.h")).read()
    assert re.search(r"#define GATO_NOALLOC_SCRATCH_BYTES \(64u << 20\)", text)
    assert ops.NOALLOC_SCRATCH_BYTES == 64 << 20
    al = (ctypes.c_float * 8)(*[2.0 ** -i for i in range(8)])
    f = lib.gato_sqp_step_noalloc
    for dims in ((14, 7, 128, 512), (14, 7, 1024, 64), (24, 12, 200, 256)):
        assert ops.gato_workspace_bytes(dims) > ops.NOALLOC_SCRATCH_BYTES
        assert f(ctypes.byref(ops.Dims(*dims)), *[None] * 9, 1e-6, 200, al, 8, 1.0, *[None] * 8, None) == \
            ops.E_WORKSPACE, dims
    assert f(ctypes.byref(ops.Dims(14, 7, 128, 0)), *[None] * 9, 1e-6, 200, al, 8, 1.0, *[None] * 8, None) == ops.OK
    assert f(ctypes.byref(ops.Dims(29, 7, 128, 4)), *[None] * 9, 1e-6, 200, al, 8, 1.0, *[None] * 8,
             None) == ops.E_UNSUPPORTED


def test_binding_argument_counts_match_the_header(lib):
    """ops.py declares as many ctypes arguments as the header has parameters."""
    protos = _prototypes()
    for fn in _declared():
        assert len(getattr(lib, fn).argtypes) == len(protos[fn]), fn


def test_library_reads_no_environment():
    """Every choice that changes which kernel or pass runs is a call argument: the
    library's sources read no environment variable."""
    csrc = os.path.join(ROOT, "block_tridiagonal_pcg_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".inc", ".cpp")):
            text = open(os.path.join(csrc, f)).read()
            assert "getenv" not in text and "environ" not in text, f


def test_library_exports_every_declared_symbol(lib):
    from block_tridiagonal_pcg_amd import ops

    for name in _declared():
        assert hasattr(lib, name), name
    assert set(ops.EXPORTS) == set(_declared())


def test_status_strings(lib):
    from block_tridiagonal_pcg_amd import ops

    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert ops.status_string(code) and ops.status_string(code) != "unknown status code"
    assert ops.status_string(12345) == "unknown status code"


def test_shapes_and_workspace(lib):
    from block_tridiagonal_pcg_amd import ops

    for n, m, N in ((14, 7, 64), (12, 6, 32), (24, 12, 16), (4, 2, 8), (14, 7, 128), (1, 1, 2), (14, 7, 1),
                    (14, 7, 1024), (24, 12, 200)):
        assert ops.gato_shape_supported(n, m, N), (n, m, N)
    for n, m, N in ((14, 7, 0), (14, 7, 1025), (24, 12, 1025), (29, 5, 10), (10, 15, 10), (0, 1, 4)):
        assert not ops.gato_shape_supported(n, m, N), (n, m, N)
    assert ops.gato_workspace_bytes((14, 7, 64, 128)) == 0          # fused: no workspace
    ws = ops.gato_workspace_bytes((14, 7, 128, 512))
    # the stage-1 outputs the direct solves read (S, gamma, Qinv, Rinv; no Phi^-1) and the
    # merit's per-knot values (17 per knot), each 256-byte aligned, then the larger of the
    # two solves' workspaces
    a = lambda x: (x * 4 + 255) // 256 * 256  # noqa: E731
    B, N = 512, 128
    stage1 = a(B * N * 3 * 14 * 14) + a(B * 17 * N) + a(B * N * 14) + a(B * N * 14 * 14) + a(B * (N - 1) * 7 * 7)
    solve = max(ops.gato_direct_workspace_bytes((14, 7, N, B)), ops.gato_cr_workspace_bytes((14, 7, N, B)))
    # the refinement pass: the correction system's q, r, e, x0, the terms h_k and t_k of its
    # gamma, then its lambda, dz and flags
    refine = a(B * N * 14) + a(B * (N - 1) * 7) + a(B * (N - 1) * 14) + a(B * 14) + 2 * a(B * N * 14) + \
        a(B * N * 14) + a(B * (N * 14 + (N - 1) * 7)) + a(B)
    assert ws == stage1 + solve + refine
    assert ops.gato_workspace_bytes((29, 7, 64, 128)) == 0          # unsupported -> 0


def test_shapes_served_by_padding(lib):
    """A shape without kernels: gato_sqp_step runs it inside the smallest compiled shape
    that holds it (2 from gato_shape_supported), with the padded copies in its workspace
    even on the fused path; the stage calls take only compiled shapes."""
    from block_tridiagonal_pcg_amd import ops

    assert ops.gato_shape_supported(14, 7, 64) == 1 and ops.gato_shape_supported(28, 14, 16) == 1
    for n, m in ((10, 5), (13, 7), (3, 1), (16, 8), (20, 10), (26, 13), (28, 1), (12, 12)):
        assert ops.gato_shape_supported(n, m, 30) == 2, (n, m)
    # the padded copies: Q, q, R, r, A, Bu, e, x0, lambda, dz in the (12, 6) shape, each 256-byte aligned
    a = lambda x: (x * 4 + 255) // 256 * 256  # noqa: E731
    B, N, n, m = 8, 32, 12, 6
    pads = a(B * N * n * n) + a(B * N * n) + a(B * (N - 1) * m * m) + a(B * (N - 1) * m) + \
        a(B * (N - 1) * n * n) + a(B * (N - 1) * n * m) + a(B * (N - 1) * n) + a(B * n) + a(B * N * n) + \
        a(B * (N * n + (N - 1) * m))
    assert ops.gato_workspace_bytes((10, 5, 32, 8)) == pads  # fused at (12, 6): nothing more
    assert ops.gato_workspace_bytes((10, 5, 100, 4)) > ops.gato_workspace_bytes((12, 6, 100, 4))
    assert ops.gato_step_solver((10, 5, 32, 8)) == ops.SOLVER_FUSED_PCG
    assert ops.gato_step_solver((18, 9, 16, 8)) == ops.SOLVER_FUSED_PCG
    assert ops.gato_step_solver((18, 9, 17, 8)) != ops.SOLVER_FUSED_PCG
    good = [ctypes.c_void_p(4096 * (j + 1)) for j in range(15)]
    assert _call_form(lib, ops.Dims(10, 5, 32, 2), good) == ops.E_UNSUPPORTED
    # the step checks its workspace for the padded layout before anything runs
    al = (ctypes.c_float * 8)(*[2.0 ** -i for i in range(8)])
    P = [ctypes.c_void_p(4096 * (j + 1)) for j in range(17)]
    args = [*P[:9], 1e-6, 200, al, 8, 1.0, *P[9:17]]
    h = lib.gato_sqp_step
    d = ops.Dims(10, 5, 32, 8)
    assert h(ctypes.byref(d), *args, None, ctypes.c_size_t(0), None, None) == ops.E_WORKSPACE
    assert h(ctypes.byref(d), *args, ctypes.c_void_p(1 << 20), ctypes.c_size_t(pads - 1), None, None) == \
        ops.E_WORKSPACE
    assert h(ctypes.byref(d), *args, ctypes.c_void_p((1 << 20) + 4), ctypes.c_size_t(pads), None, None) == ops.E_ALIGN


def test_step_workspace_for_explicit_solvers(lib):
    """An explicit direct solver runs at every horizon, the fused ones included, and needs
    the direct path's workspace there (gato_step_workspace_bytes); without one, or with too
    little, gato_sqp_step_opts returns GATO_E_WORKSPACE before anything runs."""
    from block_tridiagonal_pcg_amd import ops

    for dims in ((14, 7, 64, 128), (14, 7, 128, 512), (24, 12, 16, 8), (10, 5, 32, 8), (10, 5, 100, 4), (4, 2, 8, 1)):
        assert ops.gato_step_workspace_bytes(dims) == ops.gato_workspace_bytes(dims), dims
        assert ops.gato_step_workspace_bytes(dims, solver=ops.SOLVER_AUTO, refine=0) == \
            ops.gato_workspace_bytes(dims), dims
    # beyond the fused horizon every solver uses the same layout
    for s in (ops.SOLVER_THOMAS, ops.SOLVER_CR, ops.SOLVER_CR_STREAM):
        assert ops.gato_step_workspace_bytes((14, 7, 128, 512), solver=s) == ops.gato_workspace_bytes((14, 7, 128, 512))
    # within it, the direct path's layout where the fused path needs none: the one of a
    # horizon beyond, scaled to these dims (stage-1 rows, the solves' workspace, refinement)
    fused = (14, 7, 64, 128)
    need = ops.gato_step_workspace_bytes(fused, solver=ops.SOLVER_CR)
    assert ops.gato_workspace_bytes(fused) == 0 and need > 0
    assert need == ops.gato_step_workspace_bytes(fused, solver=ops.SOLVER_THOMAS)
    assert need >= max(ops.gato_direct_workspace_bytes(fused), ops.gato_cr_workspace_bytes(fused))
    # a padded shape adds the inner call's direct workspace to its padded copies
    assert ops.gato_step_workspace_bytes((10, 5, 32, 8), solver=ops.SOLVER_CR) == \
        ops.gato_workspace_bytes((10, 5, 32, 8)) + ops.gato_step_workspace_bytes((12, 6, 32, 8), solver=ops.SOLVER_CR)
    assert ops.gato_step_workspace_bytes((29, 7, 64, 8), solver=ops.SOLVER_CR) == 0   # unsupported
    assert ops.gato_step_workspace_bytes((14, 7, 64, 0), solver=ops.SOLVER_CR) == 0   # empty batch
    assert ops.gato_step_workspace_bytes(fused, solver=ops.SOLVER_FUSED_PCG) == 0    # rejected choices
    assert ops.gato_step_workspace_bytes(fused, solver=7) == 0
    assert ops.gato_step_workspace_bytes(fused, solver=ops.SOLVER_CR, refine=2) == 0
    al = (ctypes.c_float * 8)(*[2.0 ** -i for i in range(8)])
    P = [ctypes.c_void_p(4096 * (j + 1)) for j in range(17)]
    args = [*P[:9], 1e-6, 200, al, 8, 1.0, *P[9:17]]
    h = lib.gato_sqp_step_opts
    for dims in (fused, (10, 5, 32, 8)):
        d = ops.Dims(*dims)
        o = ops.StepOpts(ops.SOLVER_CR, 1)
        nb = ops.gato_step_workspace_bytes(dims, solver=ops.SOLVER_CR)
        assert h(ctypes.byref(d), *args, None, ctypes.c_size_t(0), None, ctypes.byref(o), None) == ops.E_WORKSPACE
        assert h(ctypes.byref(d), *args, ctypes.c_void_p(1 << 20), ctypes.c_size_t(nb - 1), None, ctypes.byref(o),
                 None) == ops.E_WORKSPACE
        assert h(ctypes.byref(d), *args, ctypes.c_void_p((1 << 20) + 4), ctypes.c_size_t(nb), None, ctypes.byref(o),
                 None) == ops.E_ALIGN


def _call_form(lib, dims, ptrs):
    d = ctypes.byref(dims) if dims is not None else None
    return lib.gato_form_schur(d, *ptrs, None)


def test_validation_happens_before_any_launch(lib):
    """Bad arguments return negative codes without touching a GPU (none is present here)."""
    from block_tridiagonal_pcg_amd import ops

    good = [ctypes.c_void_p(4096 * (j + 1)) for j in range(15)]
    d = ops.Dims(14, 7, 64, 2)
    assert _call_form(lib, None, good) == ops.E_NULL
    assert _call_form(lib, ops.Dims(14, 7, 0, 2), good) == ops.E_DIMS
    assert _call_form(lib, ops.Dims(29, 7, 64, 2), good) == ops.E_UNSUPPORTED
    bad = list(good)
    bad[0] = None
    assert _call_form(lib, d, bad) == ops.E_NULL
    bad = list(good)
    bad[3] = ctypes.c_void_p(4096 + 2)
    assert _call_form(lib, d, bad) == ops.E_ALIGN
    # B = 0: nothing to do, and nothing is launched
    assert _call_form(lib, ops.Dims(14, 7, 64, 0), good) == ops.OK

    P = [ctypes.c_void_p(4096 * (j + 1)) for j in range(17)]
    f = lib.gato_pcg_solve
    # eps <= 0 and max_iters < 1
    assert f(ctypes.byref(d), *P[:9], 0.0, 10, *P[9:14], None) == ops.E_PARAM
    assert f(ctypes.byref(d), *P[:9], 1e-6, 0, *P[9:14], None) == ops.E_PARAM
    assert f(ctypes.byref(ops.Dims(14, 7, 64, 0)), *P[:9], 1e-6, 10, *P[9:14], None) == ops.OK
    # A is not read, but a pointer given must still be aligned
    misA = list(P)
    misA[5] = ctypes.c_void_p(4096 * 6 + 2)
    assert f(ctypes.byref(d), *misA[:9], 1e-6, 10, *misA[9:14], None) == ops.E_ALIGN
    # PCG holds at most four knots per lane group
    assert f(ctypes.byref(ops.Dims(14, 7, 257, 2)), *P[:9], 1e-6, 10, *P[9:14], None) == ops.E_UNSUPPORTED

    # direct solve: workspace size, alignment and presence are checked on the host
    dd = lib.gato_direct_solve
    need = lib.gato_direct_workspace_bytes(ctypes.byref(d))
    assert need == ((2 * 64 * 14 * 15 * 4 + 255) // 256) * 256  # B=2 N=64 n=14: H^-1 rows and g
    ws = ctypes.c_void_p(1 << 20)
    assert dd(ctypes.byref(d), *P[:10], None, ctypes.c_size_t(need), None) == ops.E_WORKSPACE
    assert dd(ctypes.byref(d), *P[:10], ws, ctypes.c_size_t(need - 1), None) == ops.E_WORKSPACE
    assert dd(ctypes.byref(d), *P[:10], ctypes.c_void_p((1 << 20) + 4), ctypes.c_size_t(need), None) == ops.E_ALIGN
    assert dd(ctypes.byref(d), None, *P[1:10], ws, ctypes.c_size_t(need), None) == ops.E_NULL
    assert dd(ctypes.byref(ops.Dims(14, 7, 64, 0)), *P[:10], None, ctypes.c_size_t(0), None) == ops.OK
    assert dd(ctypes.byref(ops.Dims(5, 2, 64, 4)), *P[:10], ws, ctypes.c_size_t(need), None) == ops.E_UNSUPPORTED

    # cyclic reduction: the same host checks
    cr = lib.gato_cr_solve
    need = lib.gato_cr_workspace_bytes(ctypes.byref(d))
    # B=2 N=64 n=14: the nested dissection's interior factors (14 rows [W1 | w3] of 16
    # floats and C''s 105-entry upper triangle, padded to 108, per knot), rows of 44
    # floats for the 128 boundary knots and that system's parked rows of 16 floats (64
    # per solve); more than the streaming kernel's 44-float rows for the N knots
    assert need == ((2 * (64 * (14 * 16 + 108) + 128 * 14 * 44 + 64 * 14 * 16) * 4 + 255) // 256) * 256
    # N=1024 B=1: the streaming kernel's rows, 44 floats per knot row, are the larger layout
    long = lib.gato_cr_workspace_bytes(ctypes.byref(ops.Dims(14, 7, 1024, 1)))
    assert long == ((1024 * 14 * 44 * 4 + 255) // 256) * 256
    assert cr(ctypes.byref(d), *P[:10], None, ctypes.c_size_t(need), None) == ops.E_WORKSPACE
    assert cr(ctypes.byref(d), *P[:10], ws, ctypes.c_size_t(need - 1), None) == ops.E_WORKSPACE
    assert cr(ctypes.byref(d), *P[:10], ctypes.c_void_p((1 << 20) + 4), ctypes.c_size_t(need), None) == ops.E_ALIGN
    assert cr(ctypes.byref(d), *P[:9], None, ws, ctypes.c_size_t(need), None) == ops.E_NULL
    assert cr(ctypes.byref(ops.Dims(14, 7, 64, 0)), *P[:10], None, ctypes.c_size_t(0), None) == ops.OK
    assert cr(ctypes.byref(ops.Dims(5, 2, 64, 4)), *P[:10], ws, ctypes.c_size_t(need), None) == ops.E_UNSUPPORTED
    assert cr(ctypes.byref(ops.Dims(14, 7, 1025, 1)), *P[:10], ws, ctypes.c_size_t(1 << 40), None) == ops.E_UNSUPPORTED

    al = (ctypes.c_float * 8)(*[2.0 ** -i for i in range(8)])
    g = lib.gato_merit_eval
    assert g(ctypes.byref(d), *P[:9], al, 0, 1.0, *P[9:13], None) == ops.E_PARAM
    assert g(ctypes.byref(d), *P[:9], al, 17, 1.0, *P[9:13], None) == ops.E_PARAM
    assert g(ctypes.byref(d), *P[:9], al, 8, -1.0, *P[9:13], None) == ops.E_PARAM
    assert g(ctypes.byref(d), *P[:9], None, 8, 1.0, *P[9:13], None) == ops.E_NULL
    gs = lib.gato_merit_eval_shape
    assert gs(ctypes.byref(d), *P[:9], al, 8, 1.0, *P[9:13], 2, 0, None) == ops.E_PARAM   # unknown variant
    assert gs(ctypes.byref(d), *P[:9], al, 8, 1.0, *P[9:13], 0, 17, None) == ops.E_PARAM  # waves > 16
    assert gs(ctypes.byref(d), *P[:9], al, 8, 1.0, *P[9:13], 1, -1, None) == ops.E_PARAM  # waves < 0
    assert gs(ctypes.byref(ops.Dims(14, 7, 64, 0)), *P[:9], al, 8, 1.0, *P[9:13], 1, 4, None) == ops.OK

    h = lib.gato_sqp_step
    long_d = ops.Dims(14, 7, 128, 4)
    args = [*P[:9], 1e-6, 200, al, 8, 1.0, *P[9:17]]
    # the long-horizon path needs a workspace
    assert h(ctypes.byref(long_d), *args, None, ctypes.c_size_t(0), None, None) == ops.E_WORKSPACE
    small = ctypes.c_size_t(ops.gato_workspace_bytes((14, 7, 128, 4)) - 1)
    assert h(ctypes.byref(long_d), *args, ctypes.c_void_p(1 << 20), small, None, None) == ops.E_WORKSPACE
    ok_size = ctypes.c_size_t(ops.gato_workspace_bytes((14, 7, 128, 4)))
    assert h(ctypes.byref(long_d), *args, ctypes.c_void_p((1 << 20) + 4), ok_size, None, None) == ops.E_ALIGN
    assert h(ctypes.byref(ops.Dims(14, 7, 128, 0)), *args, None, ctypes.c_size_t(0), None, None) == ops.OK
    # gato_sqp_step_opts: the same checks, and its choices are validated first
    ho = lib.gato_sqp_step_opts
    for solver, refine in ((0, 1), (4, 1), (-2, 0), (-1, 2), (2, -1)):
        o = ops.StepOpts(solver, refine)
        assert ho(ctypes.byref(long_d), *args, ctypes.c_void_p(1 << 20), ok_size, None, ctypes.byref(o),
                  None) == ops.E_PARAM, (solver, refine)
    o = ops.StepOpts(ops.SOLVER_THOMAS, 0)
    assert ho(ctypes.byref(long_d), *args, None, ctypes.c_size_t(0), None, ctypes.byref(o), None) == ops.E_WORKSPACE
    assert ho(ctypes.byref(ops.Dims(14, 7, 128, 0)), *args, None, ctypes.c_size_t(0), None, ctypes.byref(o),
              None) == ops.OK
    assert ho(ctypes.byref(ops.Dims(14, 7, 128, 0)), *args, None, ctypes.c_size_t(0), None, None, None) == ops.OK


def test_single_knot_allows_empty_dynamics(lib):
    """With N = 1 there are no dynamics, so R, r, A, Bu, e and Rinv may be NULL."""
    from block_tridiagonal_pcg_amd import ops

    ptr = lambda j: ctypes.c_void_p(4096 * (j + 1))  # noqa: E731
    args = [ptr(0), ptr(1), None, None, None, None, None, ptr(7), None, ptr(9), ptr(10), ptr(11), ptr(12),
            None, ptr(14)]
    # B = 0 returns before any pointer is looked at
    assert lib.gato_form_schur(ctypes.byref(ops.Dims(14, 7, 1, 0)), *args, None) == ops.OK
    assert lib.gato_form_schur(ctypes.byref(ops.Dims(14, 7, 2, 0)), *args, None) == ops.OK
    # with dynamics present (N > 1) the NULL arrays are rejected before any launch; the
    # N = 1 acceptance path launches kernels, so it is exercised by the GPU tests
    assert lib.gato_form_schur(ctypes.byref(ops.Dims(14, 7, 2, 1)), *args, None) == ops.E_NULL


def test_cyclic_reduction_depth_matches_the_plan(lib):
    """The library's level count is the oracle's cyclic-frames plan length,
    ceil(log2 N) + 1, over the whole supported horizon range."""
    import oracle
    from block_tridiagonal_pcg_amd import ops

    assert ops.gato_cr_levels(0) == 0
    for N in list(range(1, 300)) + [511, 512, 513, 1023, 1024]:
        assert ops.gato_cr_levels(N) == len(oracle.cyclic_plan(N)), N


def test_horizon_policy_picks_the_measured_solver(lib):
    """Fused PCG where a workgroup holds the horizon; beyond, cyclic reduction while
    its batch time (0.18 us + 1.9 ns per knot per solve with the nested dissection,
    17 ns per knot and solve streaming for n > 16) stays below block Thomas's (2.7 us per
    knot, or 1.5 ns per knot and solve once the batch fills the chip; 6.9 us and 5.6 ns
    for n > 16).  Where the register-resident reduction runs (n <= 16, N <= 128) it
    refines on its own factors, so the refined steps are compared, as measured:
    B (0.220 + 0.00363 N) us against 3.6 N + 0.00465 N B us for block Thomas (at N = 65
    the reduction's step took 478 us against 592 at B = 1024 and 941 against 862 at
    B = 2048; at N = 128, 1409 against 1648 at B = 2048)."""
    from block_tridiagonal_pcg_amd import ops

    F, T, C = ops.SOLVER_FUSED_PCG, ops.SOLVER_THOMAS, ops.SOLVER_CR
    cases = {(14, 7, 64, 128): F, (24, 12, 16, 4): F, (14, 7, 65, 512): C, (14, 7, 65, 1024): C,
             (14, 7, 65, 2048): T, (14, 7, 128, 512): C, (14, 7, 128, 1024): C, (14, 7, 128, 2048): C,
             (14, 7, 128, 4096): C, (14, 7, 128, 8192): T,
             (14, 7, 256, 512): C, (14, 7, 256, 1024): C, (14, 7, 256, 2048): T, (14, 7, 1024, 64): C,
             (14, 7, 1024, 1024): C, (14, 7, 1024, 2048): T, (24, 12, 100, 8): C, (24, 12, 100, 256): C, (24, 12, 100, 512): T, (24, 12, 100, 1024): T}
    for dims, want in cases.items():
        assert ops.gato_step_solver(dims) == want, dims
    with pytest.raises(ops.GatoError):
        ops.gato_step_solver((29, 7, 128, 16))
