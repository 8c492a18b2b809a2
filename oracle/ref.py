"""ctypes marshalling for the fp64 C oracle (test infrastructure only).

Every function takes the problem arrays as numpy arrays in the batch-major
layouts of ``gato_oracle.c`` (any float dtype; they are upcast to float64
here), allocates float64 outputs and returns them in a dict.  No arithmetic of
the method is done in Python.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

FLAG_Q_NOT_SPD = 1
FLAG_R_NOT_SPD = 2
FLAG_S_NOT_SPD = 4
FLAG_PCG_MAXITER = 8
FLAG_PCG_BREAKDOWN = 16
FLAG_LS_FAILED = 32
FLAG_NONFINITE = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gato_oracle.c")
_LIB = os.path.join(_HERE, "libgato_oracle.so")
_lock = threading.Lock()
_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("m", ctypes.c_int), ("N", ctypes.c_int), ("B", ctypes.c_int)]


# gcc flags of the oracle build: OpenMP over solves, no fast-math (no reassociation)
CFLAGS = ("-O2", "-fopenmp", "-fno-fast-math")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (CFLAGS)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def configure(lib):
    """Set argument and return types on a loaded oracle library."""
    P = ctypes.c_void_p
    D = ctypes.c_double
    I = ctypes.c_int
    lib.gato_ref_form_schur.argtypes = [P] + [P] * 15
    lib.gato_ref_pcg_solve.argtypes = [P] + [P] * 9 + [D, I] + [P] * 5
    lib.gato_ref_merit_eval.argtypes = [P] + [P] * 10 + [I, D] + [P] * 4
    lib.gato_ref_sqp_step.argtypes = [P] + [P] * 9 + [D, I, P, I, D] + [P] * 8
    lib.gato_ref_direct_solve.argtypes = [P, P, P, P, P]
    lib.gato_ref_recover.argtypes = [P] * 9
    lib.gato_ref_num_threads.argtypes = []
    lib.gato_ref_set_num_threads.argtypes = [I]
    for f in ("gato_ref_form_schur", "gato_ref_pcg_solve", "gato_ref_merit_eval",
              "gato_ref_sqp_step", "gato_ref_direct_solve", "gato_ref_recover",
              "gato_ref_num_threads", "gato_ref_set_num_threads"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def num_threads() -> int:
    return int(load().gato_ref_num_threads())


def set_num_threads(t: int) -> int:
    """Threads of the OpenMP loops over solves from now on; returns the new count."""
    return int(load().gato_ref_set_num_threads(int(t)))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(n, m, N, B):
    return _Dims(int(n), int(m), int(N), int(B))


def _shape(Q, R):
    B, N, n, _ = Q.shape
    m = R.shape[-1]
    return n, m, N, B


def form_schur(Q, q, R, r, A, Bu, e, x0, rho=None):
    """S, Pinv, gamma, Qinv, Rinv and per-solve flags (see ``gato_oracle.c``)."""
    n, m, N, B = _shape(Q, R)
    ins = [_f64(x) for x in (Q, q, R, r, A, Bu, e, x0)]
    rh = None if rho is None else _f64(rho)
    S = np.zeros((B, N, 3, n, n))
    Pinv = np.zeros((B, N, 3, n, n))
    gamma = np.zeros((B, N, n))
    Qinv = np.zeros((B, N, n, n))
    Rinv = np.zeros((B, max(N - 1, 0), m, m))
    flags = np.zeros(B, dtype=np.int32)
    d = _dims(n, m, N, B)
    rc = load().gato_ref_form_schur(ctypes.byref(d), *[_p(x) for x in ins], _p(rh), _p(S), _p(Pinv),
                                    _p(gamma), _p(Qinv), _p(Rinv), _p(flags))
    if rc != 0:
        raise ValueError("gato_ref_form_schur returned %d" % rc)
    return dict(S=S, Pinv=Pinv, gamma=gamma, Qinv=Qinv, Rinv=Rinv, flags=flags)


def pcg_solve(S, Pinv, gamma, Qinv, Rinv, A, Bu, q, r, eps, max_iters, lambda0=None, flags=None):
    """PCG on S lambda = gamma followed by the recovery of dz."""
    B, N, _, n, _ = S.shape
    m = Rinv.shape[-1] if Rinv.ndim == 4 else r.shape[-1]
    ins = [_f64(x) for x in (S, Pinv, gamma, Qinv, Rinv, A, Bu, q, r)]
    lam = np.zeros((B, N, n)) if lambda0 is None else _f64(lambda0).copy()
    dz = np.zeros((B, N * n + (N - 1) * m))
    iters = np.zeros(B, dtype=np.int32)
    relres = np.zeros(B)
    fl = np.zeros(B, dtype=np.int32) if flags is None else np.ascontiguousarray(flags, dtype=np.int32).copy()
    d = _dims(n, m, N, B)
    rc = load().gato_ref_pcg_solve(ctypes.byref(d), *[_p(x) for x in ins], float(eps), int(max_iters),
                                   _p(lam), _p(dz), _p(iters), _p(relres), _p(fl))
    if rc != 0:
        raise ValueError("gato_ref_pcg_solve returned %d" % rc)
    return dict(lam=lam, dz=dz, iters=iters, relres=relres, flags=fl)


def merit_eval(Q, q, R, r, A, Bu, e, x0, dz, alphas, mu, flags=None):
    """Merit at each step size, merit0, best index and flags."""
    n, m, N, B = _shape(Q, R)
    ins = [_f64(x) for x in (Q, q, R, r, A, Bu, e, x0, dz)]
    al = _f64(alphas)
    merit = np.zeros((B, al.size))
    merit0 = np.zeros(B)
    best = np.zeros(B, dtype=np.int32)
    fl = np.zeros(B, dtype=np.int32) if flags is None else np.ascontiguousarray(flags, dtype=np.int32).copy()
    d = _dims(n, m, N, B)
    rc = load().gato_ref_merit_eval(ctypes.byref(d), *[_p(x) for x in ins], _p(al), int(al.size),
                                    float(mu), _p(merit), _p(merit0), _p(best), _p(fl))
    if rc != 0:
        raise ValueError("gato_ref_merit_eval returned %d" % rc)
    return dict(merit=merit, merit0=merit0, best=best, flags=fl)


def sqp_step(Q, q, R, r, A, Bu, e, x0, rho, eps, max_iters, alphas, mu, lambda0=None):
    """The whole core: form, PCG, recovery, merit and selection."""
    n, m, N, B = _shape(Q, R)
    ins = [_f64(x) for x in (Q, q, R, r, A, Bu, e, x0)]
    rh = None if rho is None else _f64(rho)
    al = _f64(alphas)
    lam = np.zeros((B, N, n)) if lambda0 is None else _f64(lambda0).copy()
    dz = np.zeros((B, N * n + (N - 1) * m))
    merit = np.zeros((B, al.size))
    merit0 = np.zeros(B)
    best = np.zeros(B, dtype=np.int32)
    iters = np.zeros(B, dtype=np.int32)
    relres = np.zeros(B)
    fl = np.zeros(B, dtype=np.int32)
    d = _dims(n, m, N, B)
    rc = load().gato_ref_sqp_step(ctypes.byref(d), *[_p(x) for x in ins], _p(rh), float(eps),
                                  int(max_iters), _p(al), int(al.size), float(mu), _p(lam), _p(dz),
                                  _p(merit), _p(merit0), _p(best), _p(iters), _p(relres), _p(fl))
    if rc != 0:
        raise ValueError("gato_ref_sqp_step returned %d" % rc)
    return dict(lam=lam, dz=dz, merit=merit, merit0=merit0, best=best, iters=iters, relres=relres,
                flags=fl)


def direct_solve(S, gamma):
    """Exact lambda by block Cholesky of S (a check on PCG, not part of the method)."""
    B, N, _, n, _ = S.shape
    lam = np.zeros((B, N, n))
    fl = np.zeros(B, dtype=np.int32)
    d = _dims(n, 1, N, B)
    rc = load().gato_ref_direct_solve(ctypes.byref(d), _p(_f64(S)), _p(_f64(gamma)), _p(lam), _p(fl))
    if rc != 0:
        raise ValueError("gato_ref_direct_solve returned %d" % rc)
    return dict(lam=lam, flags=fl)


def cyclic_plan(T):
    """The cyclic-frames elimination order for a chain of T frames (Branch page,
    "Specializing Robotics Solvers in Warp": the elimination-plan figure of "The
    three descriptions", where cyclic frames eliminate the odd frames first and
    then every other frame of what remains; the plans table's cyclic-reduction
    row).  Returns the levels in order, each the list of frames it eliminates;
    the last level is the one frame left, solved alone.  Integer bookkeeping
    only: the exact result of any valid order is the block Cholesky solve above.
    """
    remaining = list(range(T))
    levels = []
    while len(remaining) > 1:
        levels.append(remaining[1::2])  # the second, fourth, ... frame of the current chain
        remaining = remaining[0::2]
    if remaining:
        levels.append(remaining)
    return levels


def recover(Qinv, Rinv, A, Bu, q, r, lam):
    """dz from lambda (the recovery step alone)."""
    B, N, n, _ = Qinv.shape
    m = r.shape[-1]
    dz = np.zeros((B, N * n + (N - 1) * m))
    d = _dims(n, m, N, B)
    ins = [_f64(x) for x in (Qinv, Rinv, A, Bu, q, r, lam)]
    rc = load().gato_ref_recover(ctypes.byref(d), *[_p(x) for x in ins], _p(dz))
    if rc != 0:
        raise ValueError("gato_ref_recover returned %d" % rc)
    return dz
