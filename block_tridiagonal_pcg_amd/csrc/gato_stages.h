// gato_stages.h -- the three stages of the SQP-step core as workgroup-level
// device functions (GATO paper, Sec. II-III).  Every function is called by all
// threads of a workgroup in uniform control flow; lane (slot s, row i) holds
// row i of knot w0 + s.
#pragma once

#include "gato.h"
#include "gato_dev.h"

namespace gato {

struct Params {
    const float *Q, *q, *R, *r, *A, *Bu, *e, *x0, *rho;
    float *S, *Pinv, *gamma, *Qinv, *Rinv;  // stage-1 outputs (stage-2 inputs)
    float *lambda, *dz, *relres;
    int32_t* iters;
    float *merit, *merit0;
    int32_t* best;
    int32_t* flags;
    int n, m, N, B;
    float eps;
    int max_iters;
    float mu;
    int n_alpha;
    float alphas[GATO_MAX_ALPHA];
    int win_own;  // knots owned by one form workgroup (0: the whole horizon)
};

// ------------------------------------------------------------------ indexing

struct Ix {
    int n, m, N;
    __device__ __forceinline__ size_t kn(int b, int k) const { return (size_t)b * N + k; }
    __device__ __forceinline__ size_t kd(int b, int k) const { return (size_t)b * (N - 1) + k; }
    __device__ __forceinline__ size_t Q(int b, int k, int i, int c) const { return (kn(b, k) * n + i) * n + c; }
    __device__ __forceinline__ size_t vn(int b, int k, int i) const { return kn(b, k) * n + i; }
    __device__ __forceinline__ size_t R(int b, int k, int i, int c) const { return (kd(b, k) * m + i) * m + c; }
    __device__ __forceinline__ size_t vm(int b, int k, int i) const { return kd(b, k) * m + i; }
    __device__ __forceinline__ size_t A(int b, int k, int i, int c) const { return (kd(b, k) * n + i) * n + c; }
    __device__ __forceinline__ size_t Bu(int b, int k, int i, int c) const { return (kd(b, k) * n + i) * m + c; }
    __device__ __forceinline__ size_t e(int b, int k, int i) const { return kd(b, k) * n + i; }
    __device__ __forceinline__ size_t blk(int b, int k, int s, int i, int c) const
    {
        return ((kn(b, k) * 3 + s) * n + i) * n + c;
    }
    __device__ __forceinline__ size_t nz() const { return (size_t)N * n + (size_t)(N - 1) * m; }
    __device__ __forceinline__ size_t dx(int b, int k, int i) const { return (size_t)b * nz() + (size_t)k * (n + m) + i; }
    __device__ __forceinline__ size_t du(int b, int k, int i) const
    {
        return (size_t)b * nz() + (size_t)k * (n + m) + n + i;
    }
};

// Rows of one knot's block rows of S and Phi^-1, and gamma, held by lane i.
template <class SH>
struct Rows {
    float slo[SH::NC], sd[SH::NC], sup[SH::NC];
    float plo[SH::NC], pd[SH::NC], pup[SH::NC];
    float gam;
};

template <class SH>
struct FormLds {
    float xw[SH::SLOTS][SH::NP][SH::NC + 1];  // one matrix row per lane (+1: bank spread)
    float xg[SH::SLOTS][SH::NP];
};

// ------------------------------------------------------------------ stage 1: form

// S, gamma and the stair preconditioner for knots w0 .. w0+nslot-1 of solve b
// (GATO paper Sec. II eqs. 4-6; the setup kernel of Sec. III).  The block
// formulas are those of gato.h.  Knot k needs A_{k-1}, B_{k-1} terms from knot
// k-1 and D_{k+1}^-1 from knot k+1; these cross the group boundary through LDS
// between workgroup barriers (the paper's one grid-wide synchronisation
// becomes a workgroup barrier because a workgroup holds whole horizons, or a
// window with two knots of halo before and one after).
//
// Returns the lane's rows in `out`; Q~_k^-1 and R_k^-1 rows are handed to the
// sinks as soon as they exist (parked in LDS or stored), so they are not kept
// live in registers.  `fl` gets the Q/R/S_NOT_SPD bits of this knot.
template <class SH, class SinkQ, class SinkR>
__device__ __forceinline__ void form(const Params& p, int b, int w0, int nslot, FormLds<SH>& L,
                                     Rows<SH>& out, int& fl, SinkQ sinkQ, SinkR sinkR)
{
    constexpr int NC = SH::NC, MC = SH::MC, NP = SH::NP, SL = SH::SLOTS;
    const Ix ix{p.n, p.m, p.N};
    const int n = p.n, m = p.m, N = p.N;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    const int k = w0 + s;
    const bool kv = s < nslot && k < N;
    const bool hn = kv && k < N - 1;
    const bool rowv = kv && i < n;
    const float rh = (p.rho != nullptr) ? p.rho[b] : 0.0f;

    // Q~_k^-1 (identity rows on lanes/knots outside the problem keep it finite)
    float qi[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        float v = (rowv && c < n) ? p.Q[ix.Q(b, k, i, c)] : 0.0f;
        if (c == i) v = rowv ? v + rh : 1.0f;
        qi[c] = v;
    }
    bool badq = false;
    gj_steps<NP, NC>(qi, i, badq);
    sinkQ(qi);

    // R_k^-1
    float ri[MC];
#pragma unroll
    for (int c = 0; c < MC; ++c) {
        float v = (hn && i < m && c < m) ? p.R[ix.R(b, k, i, c)] : 0.0f;
        if (c == i) v = (hn && i < m) ? v : 1.0f;
        ri[c] = v;
    }
    bool badr = false;
    gj_steps<NP, MC>(ri, i, badr);
    sinkR(ri);

    // W = A_k Q~_k^-1 (row i), V = B_k R_k^-1 (row i)
    float ar[NC], W[NC], br[MC], V[MC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        ar[c] = (hn && i < n && c < n) ? p.A[ix.A(b, k, i, c)] : 0.0f;
        W[c] = 0.0f;
    }
    gemm_rows<NP, NC, NC>(W, BcRow<NP, NC>(qi), ar);
#pragma unroll
    for (int c = 0; c < MC; ++c) {
        br[c] = (hn && i < n && c < m) ? p.Bu[ix.Bu(b, k, i, c)] : 0.0f;
        V[c] = 0.0f;
    }
    gemm_rows<NP, MC, MC>(V, BcRow<NP, MC>(ri), br);

    // gamma pieces: h = (Q~_k^-1 q_k)_i (own knot), g = (e_k - W q_k - V r_k)_i (for knot k+1)
    const float qv = rowv ? p.q[ix.vn(b, k, i)] : 0.0f;
    const float rv = (hn && i < m) ? p.r[ix.vm(b, k, i)] : 0.0f;
    const float ev = (hn && i < n) ? p.e[ix.e(b, k, i)] : 0.0f;
    float h = 0.0f, t1 = 0.0f, t2 = 0.0f;
    {
        const Bc<NP> qb(qv);
        dotb<NP, NC>(h, qb, qi);
        dotb<NP, NC>(t1, qb, W);
        dotb<NP, MC>(t2, Bc<NP>(rv), V);
    }
    const float g = (ev - t1) - t2;

    // O_k = S_{k,k+1} = -W_k' (transpose through LDS); S_{k,k-1} = -W_{k-1}
    float O[NC], slo[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) L.xw[s][i][c] = W[c];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        O[c] = (i < NC) ? -L.xw[s][c][i] : 0.0f;
        slo[c] = (s >= 1 && k >= 1) ? -L.xw[s - 1][i][c] : 0.0f;
    }
    __syncthreads();

    // U_k = A_k Q~_k^-1 A_k' + B_k R_k^-1 B_k' = -(A_k O_k) + V_k B_k'
    float U[NC];
    {
        float nar[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            U[c] = 0.0f;
            nar[c] = -ar[c];
        }
        gemm_rows<NP, NC, NC>(U, BcRow<NP, NC>(O), nar);
        float bcol[NC];  // lane i < m holds column i of B_k
#pragma unroll
        for (int c = 0; c < NC; ++c) bcol[c] = (hn && i < m && c < n) ? p.Bu[ix.Bu(b, k, c, i)] : 0.0f;
        gemm_rows<NP, NC, MC>(U, BcRow<NP, NC>(bcol), V);
    }

    // D_k = Q~_k^-1 + U_{k-1};  gamma_k = h + g_{k-1}  (gamma_0 = h + x0)
#pragma unroll
    for (int c = 0; c < NC; ++c) L.xw[s][i][c] = U[c];
    L.xg[s][i] = g;
    __syncthreads();
    float sd[NC];
    float gprev = 0.0f;
    {
        const bool pv = s >= 1 && k >= 1;
#pragma unroll
        for (int c = 0; c < NC; ++c) sd[c] = pv ? qi[c] + L.xw[s - 1][i][c] : qi[c];
        gprev = pv ? L.xg[s - 1][i] : 0.0f;
    }
    __syncthreads();
    const float x0v = rowv ? p.x0[(size_t)b * n + i] : 0.0f;
    const float gam = (k >= 1) ? h + gprev : h + x0v;

    // D_k^-1
    float di[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) di[c] = sd[c];
    bool bads = false;
    gj_steps<NP, NC>(di, i, bads);

    // Phi^-1_{k,k+1} = -D_k^-1 O_k D_{k+1}^-1 ; Phi^-1_{k,k-1} = (Phi^-1_{k-1,k})'
#pragma unroll
    for (int c = 0; c < NC; ++c) L.xw[s][i][c] = di[c];
    __syncthreads();
    float Z[NC];
    {
        float Dn[NC], Y[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            Dn[c] = (s + 1 < SL) ? L.xw[s + 1][i][c] : 0.0f;
            Y[c] = 0.0f;
            Z[c] = 0.0f;
        }
        __syncthreads();
        gemm_rows<NP, NC, NC>(Y, BcRow<NP, NC>(O), di);  // Y = D_k^-1 O_k
        gemm_rows<NP, NC, NC>(Z, BcRow<NP, NC>(Dn), Y);  // Z = Y D_{k+1}^-1
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) L.xw[s][i][c] = Z[c];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        out.plo[c] = (s >= 1 && k >= 1 && i < NC) ? -L.xw[s - 1][c][i] : 0.0f;
        out.pup[c] = (k < N - 1) ? -Z[c] : 0.0f;
    }
    __syncthreads();

#pragma unroll
    for (int c = 0; c < NC; ++c) {
        out.slo[c] = rowv ? slo[c] : 0.0f;
        out.sd[c] = rowv ? sd[c] : 0.0f;
        out.sup[c] = (rowv && k < N - 1) ? O[c] : 0.0f;
        out.pd[c] = rowv ? di[c] : 0.0f;
        out.plo[c] = rowv ? out.plo[c] : 0.0f;
        out.pup[c] = rowv ? out.pup[c] : 0.0f;
    }
    out.gam = rowv ? gam : 0.0f;
    fl = 0;
    if (kv) {
        if (badq) fl |= GATO_F_Q_NOT_SPD;
        if (hn && badr) fl |= GATO_F_R_NOT_SPD;
        if (bads) fl |= GATO_F_S_NOT_SPD;
    }
}

// ------------------------------------------------------------------ stage 2: PCG

// Block-tridiagonal rows in registers (one knot per lane group).
template <class SH>
struct RegMat {
    const Rows<SH>* rw;
    __device__ __forceinline__ float S(int, float xp, float x, float xn) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        float v = 0.0f;
        dotb<NP, NC>(v, Bc<NP>(xp), rw->slo);
        dotb<NP, NC>(v, Bc<NP>(x), rw->sd);
        dotb<NP, NC>(v, Bc<NP>(xn), rw->sup);
        return v;
    }
    __device__ __forceinline__ float P(int, float xp, float x, float xn) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        float v = 0.0f;
        dotb<NP, NC>(v, Bc<NP>(xp), rw->plo);
        dotb<NP, NC>(v, Bc<NP>(x), rw->pd);
        dotb<NP, NC>(v, Bc<NP>(xn), rw->pup);
        return v;
    }
};

// Block-tridiagonal rows read from global memory at every product (for
// horizons longer than one workgroup holds); layout [B][N][3][n][n].
template <class SH>
struct GlobalMat {
    const float* Sm;
    const float* Pm;
    Ix ix;
    int b, i;
    __device__ __forceinline__ void row(const float* X, int k, int blk, float* out) const
    {
        const bool v = k < ix.N && i < ix.n;
#pragma unroll
        for (int c = 0; c < SH::NC; ++c) out[c] = (v && c < ix.n) ? X[ix.blk(b, k, blk, i, c)] : 0.0f;
    }
    __device__ __forceinline__ float mv(const float* X, int k, float xp, float x, float xn) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        float v = 0.0f, t[NC];
        row(X, k, 0, t);
        dotb<NP, NC>(v, Bc<NP>(xp), t);
        row(X, k, 1, t);
        dotb<NP, NC>(v, Bc<NP>(x), t);
        row(X, k, 2, t);
        dotb<NP, NC>(v, Bc<NP>(xn), t);
        return v;
    }
    __device__ __forceinline__ float S(int k, float xp, float x, float xn) const { return mv(Sm, k, xp, x, xn); }
    __device__ __forceinline__ float P(int k, float xp, float x, float xn) const { return mv(Pm, k, xp, x, xn); }
};

// Leaves of the canonical knot sums: at least 64 and a power of two.
__host__ __device__ constexpr int leaves_for(int knots)
{
    int p = 64;
    while (p < knots) p *= 2;
    return p;
}

template <class SH, typename RT, int C>
struct PcgLds {
    static constexpr int K = SH::SLOTS * C;     // knots held (C per lane group)
    static constexpr int P = leaves_for(K);     // canonical-sum leaves
    float xv[K][SH::NP];
    float xz[K][SH::NP];
    RT red0[P];
    RT red12[2 * P];
};

// Preconditioned CG on S lambda = gamma for one solve per workgroup (GATO
// paper Sec. II; the per-block PCG of Sec. III).  Each lane group owns C knots
// (k = c * SLOTS + s); per-knot partial sums go to LDS and every lane forms the
// same canonical total, so all waves take identical branches.  Two workgroup
// barriers per iteration: after v = S p (for p'v and v's neighbours) and after
// z = Phi^-1 r (for r'r, r'z and z's neighbours).  Each lane keeps copies of the
// neighbouring knots' entries of r and p (same row), updated with the same
// arithmetic as their owners, so the products need no further exchange.
template <class SH, typename RT, int C, class MAT>
__device__ __forceinline__ void pcg(const Params& p, const MAT& M, const float* gam, float* lam,
                                    PcgLds<SH, RT, C>& L, int& iters, float& relres, int& flags)
{
    constexpr int NP = SH::NP, SL = SH::SLOTS, KK = PcgLds<SH, RT, C>::K, P = PcgLds<SH, RT, C>::P;
    constexpr int LPL = P / 16;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    const bool lead = i == 0;
    const int nth = blockDim.x;

    for (int t = threadIdx.x; t < P; t += nth) {
        L.red0[t] = RT(0);
        L.red12[2 * t] = RT(0);
        L.red12[2 * t + 1] = RT(0);
    }
    __syncthreads();

    auto kidx = [&](int c) { return c * SL + s; };
    auto nbr = [&](float(*buf)[NP], int c, float& xp, float& xn) {
        const int kk = kidx(c);
        xp = (kk >= 1) ? buf[kk - 1][i] : 0.0f;
        xn = (kk + 1 < KK) ? buf[kk + 1][i] : 0.0f;
    };

    // ||gamma||^2 and the neighbours of lambda
    RT gg = RT(0);
    {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const RT t = groupsum<NP>(RT(gam[c]) * RT(gam[c]));
            if (lead) L.red0[kidx(c)] = t;
            L.xv[kidx(c)][i] = lam[c];
        }
        __syncthreads();
        gg = canon_sum<LPL>(L.red0);
    }
    float lp[C], ln[C];
#pragma unroll
    for (int c = 0; c < C; ++c) nbr(L.xv, c, lp[c], ln[c]);
    __syncthreads();

    iters = 0;
    flags = 0;
    if (!__builtin_isfinite(gg)) {
        flags = GATO_F_NONFINITE;
        relres = __builtin_nanf("");
        return;
    }
    if (gg == RT(0)) {
#pragma unroll
        for (int c = 0; c < C; ++c) lam[c] = 0.0f;
        relres = 0.0f;
        return;
    }
    const RT gnorm = sqrt(gg);
    const RT tol = RT(p.eps) * gnorm;
    // lambda accumulates hundreds of small steps on ill-conditioned solves; in
    // fp32 that sum alone would cost ~1e-3 of relative accuracy in dz, so it is
    // kept in fp64 (one fp64 FMA per lane per iteration) and rounded at the end.
    double lamd[C];
#pragma unroll
    for (int c = 0; c < C; ++c) lamd[c] = (double)lam[c];

    // r = gamma - S lambda, and its neighbours
    float r[C], rp[C], rn[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        r[c] = gam[c] - M.S(kidx(c), lp[c], lam[c], ln[c]);
        L.xz[kidx(c)][i] = r[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c) nbr(L.xz, c, rp[c], rn[c]);
    __syncthreads();

    // z = Phi^-1 r; r'r and r'z; neighbours of z
    float z[C], pv_[C], pp[C], pn[C];
    RT rr, rz;
    {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            z[c] = M.P(kidx(c), rp[c], r[c], rn[c]);
            const RT a = groupsum<NP>(RT(r[c]) * RT(r[c]));
            const RT bb = groupsum<NP>(RT(r[c]) * RT(z[c]));
            if (lead) {
                L.red12[2 * kidx(c)] = a;
                L.red12[2 * kidx(c) + 1] = bb;
            }
            L.xv[kidx(c)][i] = z[c];
        }
        __syncthreads();
        rr = canon_sum<LPL>(L.red12, 2);
        rz = canon_sum<LPL>(L.red12 + 1, 2);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            nbr(L.xv, c, pp[c], pn[c]);
            pv_[c] = z[c];
        }
        __syncthreads();
    }
    bool conv = sqrt(rr) <= tol;
    if (!__builtin_isfinite(rr)) flags |= GATO_F_NONFINITE;
    RT eta = rz;
    if (!conv && !(flags & GATO_F_NONFINITE)) {
        while (iters < p.max_iters) {
            // v = S p ; p'v ; v to neighbours
            float v[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                v[c] = M.S(kidx(c), pp[c], pv_[c], pn[c]);
                const RT t = groupsum<NP>(RT(pv_[c]) * RT(v[c]));
                if (lead) L.red0[kidx(c)] = t;
                L.xv[kidx(c)][i] = v[c];
            }
            __syncthreads();
            const RT pSp = canon_sum<LPL>(L.red0);
            float vp[C], vn[C];
#pragma unroll
            for (int c = 0; c < C; ++c) nbr(L.xv, c, vp[c], vn[c]);
            if (!__builtin_isfinite(pSp)) {
                flags |= GATO_F_NONFINITE;
                break;
            }
            if (!(pSp > RT(0))) {
                flags |= GATO_F_PCG_BREAKDOWN;
                break;
            }
            const float a = (float)(eta / pSp);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                lamd[c] = fma((double)a, (double)pv_[c], lamd[c]);
                r[c] = fmaf(-a, v[c], r[c]);
                rp[c] = fmaf(-a, vp[c], rp[c]);
                rn[c] = fmaf(-a, vn[c], rn[c]);
            }
            ++iters;
            // z = Phi^-1 r ; r'r, r'z ; z to neighbours
#pragma unroll
            for (int c = 0; c < C; ++c) {
                z[c] = M.P(kidx(c), rp[c], r[c], rn[c]);
                const RT ta = groupsum<NP>(RT(r[c]) * RT(r[c]));
                const RT tb = groupsum<NP>(RT(r[c]) * RT(z[c]));
                if (lead) {
                    L.red12[2 * kidx(c)] = ta;
                    L.red12[2 * kidx(c) + 1] = tb;
                }
                L.xz[kidx(c)][i] = z[c];
            }
            __syncthreads();
            rr = canon_sum<LPL>(L.red12, 2);
            const RT rz1 = canon_sum<LPL>(L.red12 + 1, 2);
            float zp[C], zn[C];
#pragma unroll
            for (int c = 0; c < C; ++c) nbr(L.xz, c, zp[c], zn[c]);
            if (!__builtin_isfinite(rr)) {
                flags |= GATO_F_NONFINITE;
                break;
            }
            if (sqrt(rr) <= tol) {
                conv = true;
                break;
            }
            if (!__builtin_isfinite(rz1)) {
                flags |= GATO_F_NONFINITE;
                break;
            }
            const float be = (float)(rz1 / eta);
            eta = rz1;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                pv_[c] = fmaf(be, pv_[c], z[c]);
                pp[c] = fmaf(be, pp[c], zp[c]);
                pn[c] = fmaf(be, pn[c], zn[c]);
            }
        }
        if (!conv && !(flags & (GATO_F_NONFINITE | GATO_F_PCG_BREAKDOWN))) flags |= GATO_F_PCG_MAXITER;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) lam[c] = (float)lamd[c];
    relres = (float)(sqrt(rr) / gnorm);
    // The loop's barriers order every LDS access above; one more before the
    // caller reuses the buffers.
    __syncthreads();
}

// ------------------------------------------------------------------ stage 2b: recovery

// dx_k = Q~_k^-1 (lambda_k - A_k' lambda_{k+1} - q_k), du_k = R_k^-1 (-B_k' lambda_{k+1} - r_k)
// (the back-substitution of the Schur solve, GATO paper Sec. II eq. 4).
template <class SH>
__device__ __forceinline__ void recover(const Params& p, int b, int k, int i, float lam, float lamn,
                                        const float* qi, const float* ri, float& dx, float& du)
{
    constexpr int NC = SH::NC, MC = SH::MC, NP = SH::NP;
    const Ix ix{p.n, p.m, p.N};
    const int n = p.n, m = p.m, N = p.N;
    const bool kv = k < N;
    const bool hn = kv && k < N - 1;
    const bool rowv = kv && i < n;
    float acol[NC], bcol[NC];
#pragma unroll
    for (int l = 0; l < NC; ++l) {
        acol[l] = (hn && i < n && l < n) ? p.A[ix.A(b, k, l, i)] : 0.0f;
        bcol[l] = (hn && i < m && l < n) ? p.Bu[ix.Bu(b, k, l, i)] : 0.0f;
    }
    const Bc<NP> lnb(lamn);
    float t = 0.0f, tb = 0.0f;
    dotb<NP, NC>(t, lnb, acol);
    dotb<NP, NC>(tb, lnb, bcol);
    const float qv = rowv ? p.q[ix.vn(b, k, i)] : 0.0f;
    const float rv = (hn && i < m) ? p.r[ix.vm(b, k, i)] : 0.0f;
    const float w = rowv ? (lam - qv) - t : 0.0f;
    const float u = (hn && i < m) ? -tb - rv : 0.0f;
    float x = 0.0f, y = 0.0f;
    dotb<NP, NC>(x, Bc<NP>(w), qi);
    dotb<NP, MC>(y, Bc<NP>(u), ri);
    dx = rowv ? x : 0.0f;
    du = (hn && i < m) ? y : 0.0f;
}

// ------------------------------------------------------------------ stage 3: merit

// Per-knot merit terms at a = 0 and at every step size (GATO paper Sec. II
// eq. 3; Sec. III eq. 7):
//   m_k(a) = a LIN + (a^2/2) QUAD + mu L1(a),
//   LIN = q'dx + r'du,  QUAD = dx'Q dx + du'R du  (undamped Q),
//   L1(a) = ||e_k + a (A dx + B du - dx_{k+1})||_1 + [k = 0] ||x0 - a dx_0||_1.
// Sums over the lanes of a group use the canonical butterfly and every rounding
// is explicit, so a knot's values do not depend on the kernel computing them.
// The group's lane 0 writes value j (j = 0: a = 0) to out[j * stride].
template <class SH>
__device__ __forceinline__ void merit_knot(const Params& p, int b, int k, int i, float dx, float du,
                                           float dxn, float* out, int stride)
{
    constexpr int NC = SH::NC, MC = SH::MC, NP = SH::NP;
    const Ix ix{p.n, p.m, p.N};
    const int n = p.n, m = p.m, N = p.N;
    const bool kv = k < N;
    const bool hn = kv && k < N - 1;
    const bool rowv = kv && i < n;
    const bool urow = hn && i < m;
    float Qr[NC], Ar[NC], Rr[MC], Br[MC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        Qr[c] = (rowv && c < n) ? p.Q[ix.Q(b, k, i, c)] : 0.0f;
        Ar[c] = (hn && i < n && c < n) ? p.A[ix.A(b, k, i, c)] : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < MC; ++c) {
        Rr[c] = (urow && c < m) ? p.R[ix.R(b, k, i, c)] : 0.0f;
        Br[c] = (hn && i < n && c < m) ? p.Bu[ix.Bu(b, k, i, c)] : 0.0f;
    }
    const float qv = rowv ? p.q[ix.vn(b, k, i)] : 0.0f;
    const float rv = urow ? p.r[ix.vm(b, k, i)] : 0.0f;
    const float ev = (hn && i < n) ? p.e[ix.e(b, k, i)] : 0.0f;
    const float x0v = (rowv && k == 0) ? p.x0[(size_t)b * n + i] : 0.0f;

    const Bc<NP> xb(dx), ub(du);
    float Qdx = 0.0f, Rdu = 0.0f, d = 0.0f;
    dotb<NP, NC>(Qdx, xb, Qr);
    dotb<NP, MC>(Rdu, ub, Rr);
    dotb<NP, NC>(d, xb, Ar);
    dotb<NP, MC>(d, ub, Br);
    d = hn ? __fsub_rn(d, dxn) : 0.0f;
    const float lin = groupsum<NP>(__fadd_rn(__fmul_rn(qv, dx), __fmul_rn(rv, du)));
    const float quad = groupsum<NP>(__fadd_rn(__fmul_rn(dx, Qdx), __fmul_rn(du, Rdu)));
    for (int j = 0; j <= p.n_alpha; ++j) {
        const float a = (j == 0) ? 0.0f : p.alphas[j - 1];
        float l1 = fabsf(__fmaf_rn(a, d, ev));
        if (k == 0) l1 = __fadd_rn(l1, fabsf(__fmaf_rn(-a, dx, x0v)));
        const float L1 = groupsum<NP>(l1);
        const float val = __fadd_rn(__fadd_rn(__fmul_rn(a, lin), __fmul_rn(__fmul_rn(0.5f, __fmul_rn(a, a)), quad)),
                                    __fmul_rn(p.mu, L1));
        if (i == 0 && kv) out[j * stride] = val;
    }
}

// Canonical sums of the per-knot merit values and the step selection
// (argmin, ties to the earlier step; accepted only below merit0).
template <int LPL>
__device__ __forceinline__ void merit_select(const Params& p, int b, const float* vals, int P, int32_t& best,
                                             int& lsfail)
{
    float M0 = canon_sum<LPL>(vals);
    float bv = 0.0f;
    int bi = 0;
    for (int j = 1; j <= p.n_alpha; ++j) {
        const float v = canon_sum<LPL>(vals + j * P);
        if (threadIdx.x == 0) p.merit[(size_t)b * p.n_alpha + (j - 1)] = v;
        if (j == 1 || v < bv) {
            bv = v;
            bi = j - 1;
        }
    }
    if (threadIdx.x == 0) p.merit0[b] = M0;
    lsfail = !(bv < M0);
    best = lsfail ? -1 : bi;
}

}  // namespace gato
