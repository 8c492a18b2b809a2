"""Thin ctypes binding of libgato.so (argument marshalling only).

The functions carry the C ABI's names and argument order.  Array arguments are
torch tensors on the GPU (float32 or int32, contiguous, in the layouts of
include/gato.h); their data pointers and the current HIP stream are passed
through unchanged.  Every step of the computation runs in the library's
kernels.  Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from ._build import LIB as _LIB_PATH

GATO_MAX_ALPHA = 16

OK = 0
E_NULL, E_DIMS, E_ALIGN, E_PARAM, E_HIP, E_UNSUPPORTED, E_WORKSPACE = -1, -2, -3, -4, -5, -6, -7

F_Q_NOT_SPD = 1
F_R_NOT_SPD = 2
F_S_NOT_SPD = 4
F_PCG_MAXITER = 8
F_PCG_BREAKDOWN = 16
F_LS_FAILED = 32
F_NONFINITE = 64

EXPORTS = (
    "gato_form_schur",
    "gato_pcg_solve",
    "gato_direct_solve",
    "gato_direct_workspace_bytes",
    "gato_cr_solve",
    "gato_cr_workspace_bytes",
    "gato_cr_levels",
    "gato_merit_eval",
    "gato_merit_eval_shape",
    "gato_sqp_step",
    "gato_sqp_step_opts",
    "gato_sqp_step_noalloc",
    "gato_workspace_bytes",
    "gato_step_workspace_bytes",
    "gato_step_solver",
    "gato_status_string",
    "gato_shape_supported",
    "gato_chain_qp",
    "gato_take_step",
)


class GatoError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__("%s failed: %s (%d)" % (fn, status_string(code), code))
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("m", ctypes.c_int32), ("N", ctypes.c_int32), ("B", ctypes.c_int32)]


class StepOpts(ctypes.Structure):
    _fields_ = [("solver", ctypes.c_int32), ("refine", ctypes.c_int32)]


class ChainParams(ctypes.Structure):
    _fields_ = [("dof", ctypes.c_int32), ("h", ctypes.c_float), ("a", ctypes.c_float), ("c", ctypes.c_float),
                ("kappa", ctypes.c_float), ("w_theta", ctypes.c_float), ("w_omega", ctypes.c_float),
                ("w_u", ctypes.c_float)]


class StageTimes(ctypes.Structure):
    _fields_ = [("schur_us", ctypes.c_float), ("linsys_us", ctypes.c_float), ("merit_us", ctypes.c_float),
                ("total_us", ctypes.c_float)]


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libgato.so (raises if it is missing: there is no fallback path)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError("libgato.so is not built (%s); run __graft_entry__.build()" % _LIB_PATH)
            lib = ctypes.CDLL(_LIB_PATH)
            P, I, F, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
            lib.gato_form_schur.argtypes = [P] * 17
            lib.gato_pcg_solve.argtypes = [P] * 10 + [F, I] + [P] * 6
            lib.gato_direct_solve.argtypes = [P] * 12 + [Z, P]
            lib.gato_direct_workspace_bytes.argtypes = [P]
            lib.gato_direct_workspace_bytes.restype = Z
            lib.gato_cr_solve.argtypes = [P] * 12 + [Z, P]
            lib.gato_cr_workspace_bytes.argtypes = [P]
            lib.gato_cr_workspace_bytes.restype = Z
            lib.gato_cr_levels.argtypes = [I]
            lib.gato_cr_levels.restype = I
            lib.gato_merit_eval.argtypes = [P] * 11 + [I, F] + [P] * 5
            lib.gato_merit_eval_shape.argtypes = [P] * 11 + [I, F] + [P] * 4 + [I, I, P]
            lib.gato_sqp_step.argtypes = [P] * 10 + [F, I, P, I, F] + [P] * 9 + [Z, P, P]
            lib.gato_sqp_step_opts.argtypes = [P] * 10 + [F, I, P, I, F] + [P] * 9 + [Z, P, P, P]
            lib.gato_sqp_step_noalloc.argtypes = [P] * 10 + [F, I, P, I, F] + [P] * 9
            lib.gato_step_solver.argtypes = [P]
            lib.gato_step_solver.restype = ctypes.c_int
            lib.gato_workspace_bytes.argtypes = [P, I]
            lib.gato_workspace_bytes.restype = Z
            lib.gato_step_workspace_bytes.argtypes = [P, I, P]
            lib.gato_step_workspace_bytes.restype = Z
            lib.gato_status_string.argtypes = [ctypes.c_int]
            lib.gato_status_string.restype = ctypes.c_char_p
            lib.gato_shape_supported.argtypes = [I, I, I]
            lib.gato_chain_qp.argtypes = [P] * 15
            lib.gato_take_step.argtypes = [P, P, I, P, P, P, P, P, F, F, P]
            for f in ("gato_form_schur", "gato_pcg_solve", "gato_direct_solve", "gato_cr_solve", "gato_merit_eval",
                      "gato_merit_eval_shape", "gato_sqp_step", "gato_sqp_step_opts", "gato_sqp_step_noalloc",
                      "gato_shape_supported", "gato_chain_qp", "gato_take_step"):
                getattr(lib, f).restype = ctypes.c_int
            _lib = lib
    return _lib


def status_string(code: int) -> str:
    return load().gato_status_string(int(code)).decode()


def _dims(n, m, N, B):
    return Dims(int(n), int(m), int(N), int(B))


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _chk(t, name, dtype=torch.float32, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _shapes(n, m, N, B):
    d = max(N - 1, 0)
    return dict(Q=(B, N, n, n), q=(B, N, n), R=(B, d, m, m), r=(B, d, m), A=(B, d, n, n), Bu=(B, d, n, m),
                e=(B, d, n), x0=(B, n), rho=(B,), S=(B, N, 3, n, n), Pinv=(B, N, 3, n, n), gamma=(B, N, n),
                Qinv=(B, N, n, n), Rinv=(B, d, m, m), lam=(B, N, n), dz=(B, N * n + d * m), B_=(B,))


def _raise(fn, rc):
    if rc != OK:
        raise GatoError(fn, rc)
    return rc


def gato_form_schur(dims, Q, q, R, r, A, Bu, e, x0, rho, S, Pinv, gamma, Qinv, Rinv, flags, stream=None):
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    for t, k in ((Q, "Q"), (q, "q"), (R, "R"), (r, "r"), (A, "A"), (Bu, "Bu"), (e, "e"), (x0, "x0"),
                 (rho, "rho"), (S, "S"), (Pinv, "Pinv"), (gamma, "gamma"), (Qinv, "Qinv"), (Rinv, "Rinv")):
        _chk(t, k, shape=sh[k])
    _chk(flags, "flags", torch.int32, sh["B_"])
    d = _dims(n, m, N, B)
    rc = load().gato_form_schur(ctypes.byref(d), _p(Q), _p(q), _p(R), _p(r), _p(A), _p(Bu), _p(e), _p(x0),
                                _p(rho), _p(S), _p(Pinv), _p(gamma), _p(Qinv), _p(Rinv), _p(flags),
                                _stream(stream))
    return _raise("gato_form_schur", rc)


def gato_pcg_solve(dims, S, Pinv, gamma, Qinv, Rinv, A, Bu, q, r, eps, max_iters, lam, dz, iters, relres,
                   flags, stream=None):
    """A may be None: the library takes A_k' from S's upper blocks and does not read it."""
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    for t, k in ((S, "S"), (Pinv, "Pinv"), (gamma, "gamma"), (Qinv, "Qinv"), (Rinv, "Rinv"), (A, "A"),
                 (Bu, "Bu"), (q, "q"), (r, "r"), (lam, "lam"), (dz, "dz"), (relres, "B_")):
        _chk(t, k, shape=sh[k])
    _chk(iters, "iters", torch.int32, sh["B_"])
    _chk(flags, "flags", torch.int32, sh["B_"])
    d = _dims(n, m, N, B)
    rc = load().gato_pcg_solve(ctypes.byref(d), _p(S), _p(Pinv), _p(gamma), _p(Qinv), _p(Rinv), _p(A), _p(Bu),
                               _p(q), _p(r), float(eps), int(max_iters), _p(lam), _p(dz), _p(iters),
                               _p(relres), _p(flags), _stream(stream))
    return _raise("gato_pcg_solve", rc)


def gato_direct_workspace_bytes(dims):
    return int(load().gato_direct_workspace_bytes(ctypes.byref(_dims(*dims))))


def direct_workspace_for(dims, device="cuda"):
    nb = gato_direct_workspace_bytes(dims)
    return torch.empty(nb, dtype=torch.uint8, device=device) if nb > 0 else None


def gato_direct_solve(dims, S, gamma, Qinv, Rinv, Bu, q, r, lam, dz, flags, workspace, stream=None):
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    for t, k in ((S, "S"), (gamma, "gamma"), (Qinv, "Qinv"), (Rinv, "Rinv"), (Bu, "Bu"), (q, "q"), (r, "r"),
                 (lam, "lam"), (dz, "dz")):
        _chk(t, k, shape=sh[k])
    _chk(flags, "flags", torch.int32, sh["B_"])
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _chk(workspace, "workspace", torch.uint8)
        ws_ptr, ws_bytes = _p(workspace), workspace.numel()
    d = _dims(n, m, N, B)
    rc = load().gato_direct_solve(ctypes.byref(d), _p(S), _p(gamma), _p(Qinv), _p(Rinv), _p(Bu), _p(q), _p(r),
                                  _p(lam), _p(dz), _p(flags), ws_ptr, ctypes.c_size_t(ws_bytes), _stream(stream))
    return _raise("gato_direct_solve", rc)


def gato_cr_workspace_bytes(dims):
    return int(load().gato_cr_workspace_bytes(ctypes.byref(_dims(*dims))))


def cr_workspace_for(dims, device="cuda"):
    nb = gato_cr_workspace_bytes(dims)
    return torch.empty(nb, dtype=torch.uint8, device=device) if nb > 0 else None


def gato_cr_levels(N):
    return int(load().gato_cr_levels(int(N)))


def gato_cr_solve(dims, S, gamma, Qinv, Rinv, Bu, q, r, lam, dz, flags, workspace, stream=None):
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    for t, k in ((S, "S"), (gamma, "gamma"), (Qinv, "Qinv"), (Rinv, "Rinv"), (Bu, "Bu"), (q, "q"), (r, "r"),
                 (lam, "lam"), (dz, "dz")):
        _chk(t, k, shape=sh[k])
    _chk(flags, "flags", torch.int32, sh["B_"])
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _chk(workspace, "workspace", torch.uint8)
        ws_ptr, ws_bytes = _p(workspace), workspace.numel()
    d = _dims(n, m, N, B)
    rc = load().gato_cr_solve(ctypes.byref(d), _p(S), _p(gamma), _p(Qinv), _p(Rinv), _p(Bu), _p(q), _p(r),
                              _p(lam), _p(dz), _p(flags), ws_ptr, ctypes.c_size_t(ws_bytes), _stream(stream))
    return _raise("gato_cr_solve", rc)


SOLVER_AUTO, SOLVER_FUSED_PCG, SOLVER_THOMAS, SOLVER_CR, SOLVER_CR_STREAM = -1, 0, 1, 2, 3
MERIT_PER_KNOT, MERIT_PER_CANDIDATE = 0, 1


def gato_step_solver(dims):
    """The stage-2 solver gato_sqp_step runs for dims (the library's horizon policy)."""
    rc = int(load().gato_step_solver(ctypes.byref(_dims(*dims))))
    if rc < 0:
        raise GatoError("gato_step_solver", rc)
    return rc


def _alphas(alphas):
    a = [float(x) for x in alphas]
    arr = (ctypes.c_float * max(len(a), 1))(*a)
    return arr, len(a)


def gato_merit_eval(dims, Q, q, R, r, A, Bu, e, x0, dz, alphas, mu, merit, merit0, best, flags, stream=None,
                    variant=None, waves=0):
    """With variant None, gato_merit_eval; else gato_merit_eval_shape with that launch
    variant (MERIT_PER_KNOT / MERIT_PER_CANDIDATE) and `waves` wavefronts per workgroup."""
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    for t, k in ((Q, "Q"), (q, "q"), (R, "R"), (r, "r"), (A, "A"), (Bu, "Bu"), (e, "e"), (x0, "x0"),
                 (dz, "dz"), (merit0, "B_")):
        _chk(t, k, shape=sh[k])
    arr, na = _alphas(alphas)
    _chk(merit, "merit", shape=(B, na))
    _chk(best, "best", torch.int32, sh["B_"])
    _chk(flags, "flags", torch.int32, sh["B_"])
    d = _dims(n, m, N, B)
    args = (ctypes.byref(d), _p(Q), _p(q), _p(R), _p(r), _p(A), _p(Bu), _p(e), _p(x0), _p(dz), arr, na, float(mu),
            _p(merit), _p(merit0), _p(best), _p(flags))
    if variant is None:
        return _raise("gato_merit_eval", load().gato_merit_eval(*args, _stream(stream)))
    rc = load().gato_merit_eval_shape(*args, int(variant), int(waves), _stream(stream))
    return _raise("gato_merit_eval_shape", rc)


def gato_workspace_bytes(dims, n_alpha=8):
    d = _dims(*dims)
    return int(load().gato_workspace_bytes(ctypes.byref(d), int(n_alpha)))


def gato_step_workspace_bytes(dims, n_alpha=8, solver=None, refine=None):
    """Bytes of workspace gato_sqp_step_opts needs with these choices (None: gato_sqp_step's)."""
    d = _dims(*dims)
    o = _opts(solver, refine)
    return int(load().gato_step_workspace_bytes(ctypes.byref(d), int(n_alpha), ctypes.byref(o) if o else None))


def gato_shape_supported(n, m, N):
    """1: the build has kernels for (n, m); 2: gato_sqp_step serves it by padding to a
    compiled shape (the stage calls do not); 0: unsupported."""
    return int(load().gato_shape_supported(int(n), int(m), int(N)))


def _opts(solver, refine):
    if solver is None and refine is None:
        return None
    return StepOpts(SOLVER_AUTO if solver is None else int(solver), 1 if refine is None else int(refine))


def gato_sqp_step(dims, Q, q, R, r, A, Bu, e, x0, rho, eps, max_iters, alphas, mu, lam, dz, merit, merit0,
                  best, iters, relres, flags, workspace=None, times=False, stream=None, solver=None, refine=None):
    """One SQP iteration's core.  `workspace` is a uint8 CUDA tensor (or None when the
    fused path needs none); with times=True returns a StageTimes (the call synchronises).
    With solver or refine given the call is gato_sqp_step_opts with those choices."""
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    for t, k in ((Q, "Q"), (q, "q"), (R, "R"), (r, "r"), (A, "A"), (Bu, "Bu"), (e, "e"), (x0, "x0"),
                 (rho, "rho"), (lam, "lam"), (dz, "dz"), (merit0, "B_"), (relres, "B_")):
        _chk(t, k, shape=sh[k])
    arr, na = _alphas(alphas)
    _chk(merit, "merit", shape=(B, na))
    for t, k in ((best, "best"), (iters, "iters"), (flags, "flags")):
        _chk(t, k, torch.int32, sh["B_"])
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _chk(workspace, "workspace", torch.uint8)
        ws_ptr, ws_bytes = _p(workspace), workspace.numel()
    st = StageTimes() if times else None
    d = _dims(n, m, N, B)
    args = (ctypes.byref(d), _p(Q), _p(q), _p(R), _p(r), _p(A), _p(Bu), _p(e), _p(x0), _p(rho), float(eps),
            int(max_iters), arr, na, float(mu), _p(lam), _p(dz), _p(merit), _p(merit0), _p(best), _p(iters),
            _p(relres), _p(flags), ws_ptr, ctypes.c_size_t(ws_bytes), ctypes.byref(st) if st is not None else None)
    o = _opts(solver, refine)
    if o is None:
        _raise("gato_sqp_step", load().gato_sqp_step(*args, _stream(stream)))
    else:
        _raise("gato_sqp_step_opts", load().gato_sqp_step_opts(*args, ctypes.byref(o), _stream(stream)))
    return st


NOALLOC_SCRATCH_BYTES = 64 << 20


def gato_sqp_step_noalloc(dims, Q, q, R, r, A, Bu, e, x0, rho, eps, max_iters, alphas, mu, lam, dz, merit, merit0,
                          best, iters, relres, flags, stream=None):
    """gato_sqp_step with the library's fixed per-device scratch array in place of a
    workspace (for callers that cannot allocate); raises GatoError(E_WORKSPACE) when
    the dims need more than NOALLOC_SCRATCH_BYTES."""
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    for t, k in ((Q, "Q"), (q, "q"), (R, "R"), (r, "r"), (A, "A"), (Bu, "Bu"), (e, "e"), (x0, "x0"),
                 (rho, "rho"), (lam, "lam"), (dz, "dz"), (merit0, "B_"), (relres, "B_")):
        _chk(t, k, shape=sh[k])
    arr, na = _alphas(alphas)
    _chk(merit, "merit", shape=(B, na))
    for t, k in ((best, "best"), (iters, "iters"), (flags, "flags")):
        _chk(t, k, torch.int32, sh["B_"])
    d = _dims(n, m, N, B)
    rc = load().gato_sqp_step_noalloc(ctypes.byref(d), _p(Q), _p(q), _p(R), _p(r), _p(A), _p(Bu), _p(e), _p(x0),
                                      _p(rho), float(eps), int(max_iters), arr, na, float(mu), _p(lam), _p(dz),
                                      _p(merit), _p(merit0), _p(best), _p(iters), _p(relres), _p(flags),
                                      _stream(stream))
    return _raise("gato_sqp_step_noalloc", rc)


# ---------------------------------------------------------------- the SQP driver's kernels


def chain_params(P):
    """The C struct of a synth.Chain's parameters."""
    return ChainParams(int(P.dof), float(P.h), float(P.a), float(P.c), float(P.kappa), float(P.w_theta),
                       float(P.w_omega), float(P.w_u))


def gato_chain_qp(dims, plant, X, U, x_init, x_ref, Q, q, R, r, A, Bu, e, x0, stream=None):
    """The chain plant's QP data at (X, U) (include/gato_driver.h); `plant` is a ChainParams."""
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    _chk(X, "X", shape=(B, N, n))
    _chk(U, "U", shape=(B, N - 1, m))
    _chk(x_init, "x_init", shape=(B, n))
    _chk(x_ref, "x_ref", shape=(B, n))
    for t, k in ((Q, "Q"), (q, "q"), (R, "R"), (r, "r"), (A, "A"), (Bu, "Bu"), (e, "e"), (x0, "x0")):
        _chk(t, k, shape=sh[k])
    d = _dims(n, m, N, B)
    rc = load().gato_chain_qp(ctypes.byref(d), ctypes.byref(plant), _p(X), _p(U), _p(x_init), _p(x_ref), _p(Q),
                              _p(q), _p(R), _p(r), _p(A), _p(Bu), _p(e), _p(x0), _stream(stream))
    return _raise("gato_chain_qp", rc)


def gato_take_step(dims, alphas, dz, best, X, U, rho, rho_min, rho_max, stream=None):
    """X += a dX, U += a dU with a = alphas[best] (0 on a failed line search), and the
    damping update (include/gato_driver.h)."""
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    _chk(dz, "dz", shape=sh["dz"])
    _chk(best, "best", torch.int32, sh["B_"])
    _chk(X, "X", shape=(B, N, n))
    _chk(U, "U", shape=(B, N - 1, m))
    _chk(rho, "rho", shape=(B,))
    arr, na = _alphas(alphas)
    d = _dims(n, m, N, B)
    rc = load().gato_take_step(ctypes.byref(d), arr, na, _p(dz), _p(best), _p(X), _p(U), _p(rho), float(rho_min),
                               float(rho_max), _stream(stream))
    return _raise("gato_take_step", rc)


# ---------------------------------------------------------------- allocation helpers


def to_device(batch, device="cuda"):
    """Copy a synth batch (numpy float32 arrays) to the GPU as contiguous tensors."""
    fields = ("Q", "q", "R", "r", "A", "Bu", "e", "x0")
    out = {k: torch.from_numpy(batch[k]).to(device).contiguous() for k in fields}
    out["dims"] = batch["dims"]
    return out


def workspace_for(dims, n_alpha=8, device="cuda", solver=None, refine=None):
    """The workspace gato_sqp_step (gato_sqp_step_opts with solver/refine) needs, or None."""
    nb = gato_step_workspace_bytes(dims, n_alpha, solver, refine)
    return torch.empty(nb, dtype=torch.uint8, device=device) if nb > 0 else None


def alloc_outputs(dims, n_alpha=8, device="cuda"):
    n, m, N, B = dims
    f32, i32 = torch.float32, torch.int32
    sh = _shapes(n, m, N, B)
    z = lambda k, dt=f32: torch.zeros(sh[k], dtype=dt, device=device)  # noqa: E731
    return dict(S=z("S"), Pinv=z("Pinv"), gamma=z("gamma"), Qinv=z("Qinv"), Rinv=z("Rinv"), lam=z("lam"),
                dz=z("dz"), merit=torch.zeros((B, n_alpha), dtype=f32, device=device), merit0=z("B_"),
                best=z("B_", i32), iters=z("B_", i32), relres=z("B_"), flags=z("B_", i32))


def prepared_sqp_step(dims, Q, q, R, r, A, Bu, e, x0, rho, eps, max_iters, alphas, mu, lam, dz, merit, merit0,
                      best, iters, relres, flags, workspace=None, stream=None, solver=None, refine=None):
    """Check and marshal gato_sqp_step's arguments once; return a callable that only
    makes the C call (for timing loops).  The tensors must stay alive and in place.
    With solver or refine given it calls gato_sqp_step_opts with those choices."""
    n, m, N, B = dims
    sh = _shapes(n, m, N, B)
    for t, k in ((Q, "Q"), (q, "q"), (R, "R"), (r, "r"), (A, "A"), (Bu, "Bu"), (e, "e"), (x0, "x0"),
                 (rho, "rho"), (lam, "lam"), (dz, "dz"), (merit0, "B_"), (relres, "B_")):
        _chk(t, k, shape=sh[k])
    arr, na = _alphas(alphas)
    _chk(merit, "merit", shape=(B, na))
    for t, k in ((best, "best"), (iters, "iters"), (flags, "flags")):
        _chk(t, k, torch.int32, sh["B_"])
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _chk(workspace, "workspace", torch.uint8)
        ws_ptr, ws_bytes = _p(workspace), workspace.numel()
    d = _dims(n, m, N, B)
    o = _opts(solver, refine)
    args = (ctypes.byref(d), _p(Q), _p(q), _p(R), _p(r), _p(A), _p(Bu), _p(e), _p(x0), _p(rho), float(eps),
            int(max_iters), arr, na, float(mu), _p(lam), _p(dz), _p(merit), _p(merit0), _p(best), _p(iters),
            _p(relres), _p(flags), ws_ptr, ctypes.c_size_t(ws_bytes), None)
    if o is None:
        fn = load().gato_sqp_step
        args = args + (_stream(stream),)
    else:
        fn = load().gato_sqp_step_opts
        args = args + (ctypes.byref(o), _stream(stream))
    keep = (d, arr, o)  # noqa: F841  (kept alive by the closure)

    def call():
        rc = fn(*args)
        if rc != OK:
            raise GatoError("gato_sqp_step", rc)
        return keep

    return call


def stage_times(dims, dev, eps, max_iters, alphas, mu, reps=10, stream=None):
    """Median device time (us) of the three standalone calls on `dev` (a to_device batch):
    gato_form_schur, stage 2 as gato_sqp_step runs it (gato_pcg_solve from a cold start
    where the fused path applies, else gato_cr_solve or gato_direct_solve as
    gato_step_solver says), gato_merit_eval."""
    import statistics

    st = torch.cuda.current_stream() if stream is None else stream
    out = alloc_outputs(dims, len(alphas))
    direct = gato_workspace_bytes(dims, len(alphas)) > 0
    cr = direct and gato_step_solver(dims) == SOLVER_CR
    dws = (cr_workspace_for(dims) if cr else direct_workspace_for(dims)) if direct else None
    fields = ("Q", "q", "R", "r", "A", "Bu", "e", "x0")
    res = {"schur_us": [], "linsys_us": [], "merit_us": []}
    for _ in range(reps + 1):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record(st)
        gato_form_schur(dims, *[dev[f] for f in fields], None, out["S"], out["Pinv"], out["gamma"], out["Qinv"],
                        out["Rinv"], out["flags"], stream=st)
        ev[1].record(st)
        out["lam"].zero_()
        ev[2].record(st)
        if cr:
            gato_cr_solve(dims, out["S"], out["gamma"], out["Qinv"], out["Rinv"], dev["Bu"], dev["q"], dev["r"],
                          out["lam"], out["dz"], out["flags"], dws, stream=st)
        elif direct:
            gato_direct_solve(dims, out["S"], out["gamma"], out["Qinv"], out["Rinv"], dev["Bu"], dev["q"], dev["r"],
                              out["lam"], out["dz"], out["flags"], dws, stream=st)
        else:
            gato_pcg_solve(dims, out["S"], out["Pinv"], out["gamma"], out["Qinv"], out["Rinv"], dev["A"], dev["Bu"],
                           dev["q"], dev["r"], eps, max_iters, out["lam"], out["dz"], out["iters"], out["relres"],
                           out["flags"], stream=st)
        ev[3].record(st)
        ev[4].record(st)
        gato_merit_eval(dims, *[dev[f] for f in fields], out["dz"], alphas, mu, out["merit"], out["merit0"],
                        out["best"], out["flags"], stream=st)
        ev[5].record(st)
        torch.cuda.synchronize()
        res["schur_us"].append(1e3 * ev[0].elapsed_time(ev[1]))
        res["linsys_us"].append(1e3 * ev[2].elapsed_time(ev[3]))
        res["merit_us"].append(1e3 * ev[4].elapsed_time(ev[5]))
    return {k: statistics.median(v[1:]) for k, v in res.items()}
