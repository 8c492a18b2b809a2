"""Dense, textbook forms of the QP for checking the oracle (numpy, tests only).

Everything here is assembled straight from the QP's definition -- cost blocks on
a block diagonal, dynamics as constraint rows -- and solved with LAPACK through
numpy.  None of it uses the Schur-complement formulas the oracle implements, so
agreement between the two is evidence about the oracle, not a restatement of it.
"""
import numpy as np


def sizes(n, m, N):
    return N * n + (N - 1) * m


def x_index(k, n, m):
    return k * (n + m)


def u_index(k, n, m):
    return k * (n + m) + n


def assemble(batch, b, rho=0.0):
    """G, g, C, c (and the undamped G0) for solve b, in float64.

    G dz = blkdiag(Q_0 + rho I, R_0, ..., Q_{N-1} + rho I); g = (q_0, r_0, ...);
    C dz = c encodes dx_0 = x0 and dx_{k+1} - A_k dx_k - B_k du_k = e_k.
    """
    n, m, N, _ = batch["dims"]
    f = {k: np.asarray(batch[k][b], dtype=np.float64) for k in ("Q", "q", "R", "r", "A", "Bu", "e", "x0")}
    nz = sizes(n, m, N)
    G0 = np.zeros((nz, nz))
    g = np.zeros(nz)
    for k in range(N):
        i = x_index(k, n, m)
        G0[i:i + n, i:i + n] = f["Q"][k]
        g[i:i + n] = f["q"][k]
        if k < N - 1:
            j = u_index(k, n, m)
            G0[j:j + m, j:j + m] = f["R"][k]
            g[j:j + m] = f["r"][k]
    G = G0.copy()
    for k in range(N):
        i = x_index(k, n, m)
        G[i:i + n, i:i + n] += rho * np.eye(n)
    C = np.zeros((N * n, nz))
    c = np.zeros(N * n)
    C[0:n, 0:n] = np.eye(n)
    c[0:n] = f["x0"]
    for k in range(N - 1):
        row = (k + 1) * n
        C[row:row + n, x_index(k, n, m):x_index(k, n, m) + n] = -f["A"][k]
        C[row:row + n, u_index(k, n, m):u_index(k, n, m) + m] = -f["Bu"][k]
        C[row:row + n, x_index(k + 1, n, m):x_index(k + 1, n, m) + n] = np.eye(n)
        c[row:row + n] = f["e"][k]
    return dict(G=G, G0=G0, g=g, C=C, c=c)


def kkt_solve(G, g, C, c):
    """Solve [[G, -C'], [C, 0]] [dz; lam] = [-g; c] by dense LU."""
    nz = G.shape[0]
    nc = C.shape[0]
    K = np.zeros((nz + nc, nz + nc))
    K[:nz, :nz] = G
    K[:nz, nz:] = -C.T
    K[nz:, :nz] = C
    rhs = np.concatenate([-g, c])
    sol = np.linalg.solve(K, rhs)
    return sol[:nz], sol[nz:]


def btd_dense(X):
    """Dense matrix from block rows [N][3][n][n] (one solve)."""
    N, _, n, _ = X.shape
    D = np.zeros((N * n, N * n))
    for k in range(N):
        for s in range(3):
            kk = k + s - 1
            if 0 <= kk < N:
                D[k * n:(k + 1) * n, kk * n:(kk + 1) * n] = X[k, s]
    return D


def merit_dense(G0, g, C, c, dz, alpha, mu):
    """alpha g'dz + alpha^2/2 dz'G0 dz + mu ||c - alpha C dz||_1 (matrix form of the merit)."""
    return alpha * g @ dz + 0.5 * alpha * alpha * dz @ G0 @ dz + mu * np.abs(c - alpha * (C @ dz)).sum()
