// gato.hip -- kernels and C ABI of libgato.so (gfx950).
//
// Kernels (one workgroup per solve unless noted):
//   k_sqp_fused   form -> PCG -> recovery -> merit -> selection, everything in
//                 registers and LDS; used when a workgroup holds the horizon.
//   k_form        stage 1 alone, one workgroup per window of knots (any N).
//   k_pcg_res     stage 2 alone with S and Phi^-1 rows loaded once into registers.
//   k_pcg_stream  stage 2 alone for horizons longer than a workgroup holds:
//                 C knots per lane group; with two (n <= 16) S's diagonal blocks
//                 and D^-1 stay on chip and only S's other blocks are re-read
//                 per product, otherwise every row is.
//   k_direct      stage 2 by block Thomas elimination, one lane group per solve.
//   k_kkt_residual, k_refine_gamma, k_refine_add
//                 the KKT refinement pass around a second direct solve (block
//                 Thomas, the streaming and nested-dissection reductions).
// Stage 2 by block cyclic reduction (k_cr, k_cr_res, k_cr_res_ref with the
// refinement pass inside) is in gato_cr.hip.
//   k_merit       stage 3 alone; any workgroup size gives identical bits.
//   k_merit_knots, k_merit_sum
//                 the same stage with a solve's knots over several workgroups
//                 (gato_sqp_step on long horizons with a small batch).
#include "gato_internal.h"
#include "gato_stages.h"

#include <algorithm>
#include <cstring>
#include <mutex>

namespace gato {

// ------------------------------------------------------------------ fused step

template <class SH>
struct FusedLds {
    Park<SH> park;  // G^-1 rows, kept for the recovery
    union {
        FormLds<SH> form;
        PcgLds<SH, 1> pcg;
        alignas(16) float mer[(GATO_MAX_ALPHA + 1) * 64];
    } u;
    int flags;
};

// VS: the PCG's stop test on the vector unit (pcg()), for launches of at most
// 512 threads, which also leaves the kernel up to 256 registers per lane.
template <class SH, bool VS>
__global__ __launch_bounds__(VS && SH::THREADS > 512 ? 512 : SH::THREADS) void k_sqp_fused(Params p)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC;
    __shared__ FusedLds<SH> L;
    const Ix<SH> ix{p.N};
    const int b = blockIdx.x;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP, k = s;
    const bool kv = k < p.N, hn = kv && k < p.N - 1, rowv = kv && i < NC;
    if (threadIdx.x == 0) L.flags = 0;

    // the starting point, loaded now so that its latency hides behind the formation
    float lam = ld1(p.lambda, ix.vn(b, k, i), rowv);
    Rows<SH> rw;
    int fl = 0;
    form<SH, true, true>(p, b, 0, p.N, L.u.form, L.park, rw, fl, [](const float*, const float*) {});
    if (fl && i == 0) atomicOr(&L.flags, fl);

    int it = 0, pfl = 0;
    float rel = 0.0f;
    const RegMat<SH> M{&rw};
    pcg_robust<SH, 1, RegMat<SH>, VS, !VS>(p, M, &rw.gam, &lam, L.u.pcg, it, rel, pfl);

    // recovery of dz (exchange rows of the PCG buffers: knot k at row k + 1)
    L.u.pcg.xv[s + 1][i] = lam;
    __syncthreads();
    const float lamn = L.u.pcg.xv[s + 2][i];
    float qi[NC], ri[MC], bc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        qi[c] = L.park.Q[s][i < NC ? i : 0][c];
        bc[c] = L.park.Bt[s][i < MC ? i : 0][c];
    }
#pragma unroll
    for (int c = 0; c < MC; ++c) ri[c] = L.park.R[s][i < MC ? i : 0][c];
    float dx, du;
    recover<SH>(i, rowv, hn && i < MC, lam, lamn, qi, rw.sup, L.park.h[s][i], bc, L.park.rv[s][i], ri, dx, du);
    if (rowv) {
        p.lambda[ix.vn(b, k, i)] = lam;
        p.dz[ix.dx(b, k, i)] = dx;
    }
    if (hn && i < MC) p.dz[ix.du(b, k, i)] = du;
    __syncthreads();

    // merit at every step size, then the selection
    L.u.pcg.xv[s + 1][i] = dx;
    __syncthreads();
    const float dxn = L.u.pcg.xv[s + 2][i];
    __syncthreads();
    for (int t = threadIdx.x; t < (GATO_MAX_ALPHA + 1) * 64; t += blockDim.x) L.u.mer[t] = 0.0f;
    __syncthreads();
    MeritIn<SH> mi;
    wave_prio<true, 3>();
    merit_rows<SH>(p, b, k, i, mi);
    wave_prio<true, 2>();
    merit_knot<SH>(p, k, i, mi, dx, du, dxn, L.u.mer + k, 64);
    wave_prio<true, 0>();
    __syncthreads();
    int32_t best;
    int lsfail;
    merit_select<4>(p, b, L.u.mer, 64, best, lsfail);
    if (threadIdx.x == 0) {
        p.iters[b] = it;
        p.relres[b] = rel;
        p.best[b] = best;
        p.flags[b] = L.flags | pfl | (lsfail ? GATO_F_LS_FAILED : 0);
    }
}

// ------------------------------------------------------------------ stage 1 alone

__global__ void k_zero_i32(int32_t* x, int count)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < count) x[t] = 0;
}

// ------------------------------------------------------------------ iterative refinement

// One pass of iterative refinement of the KKT system the Schur method solves
// (G dz - C' lambda = -g, C dz = c; GATO paper Sec. II, eq. 2): the residual of
// the first pass's (lambda, dz), accumulated in double from the problem data,
// is the right-hand side (g', c') of a correction system with the same G and
// C, whose q, r, e and x0 (kkt_rows) are q'_k, r'_k, e'_k and x0' (rows of C:
// [I] for knot 0, [-A_k, -B_k, I] for knot k + 1).  The products of
// fp32 data are exact in double and the sums nearly so, so the correction
// carries the first pass's error however ill-conditioned S is, while the fp32
// solve finds it with its usual relative accuracy.  S, Q~^-1 and R^-1 are those
// of the first pass; the correction's gamma (gamma'_0 = x0' + h_0,
// gamma'_{k+1} = e'_k - t_k + h_{k+1}, as the formation forms gamma) takes
// h_k = Q~_k^-1 q'_k and t_k = A_k h_k + B_k R_k^-1 r'_k from here.  (The
// register-resident cyclic reduction runs the whole pass inside its kernel;
// this one serves the other direct solves.)
// Lane group of NP lanes per knot, lane i: row i of each knot block; the
// vectors a row needs whole go through the group's LDS rows.
template <class SH>
__global__ __launch_bounds__(256) void k_kkt_residual(const Params p, float* qc, float* rc, float* ec, float* x0c,
                                                      float* hq, float* tq)
{
    constexpr int NP = SH::NP, n = SH::NC, m = SH::MC, G = 256 / NP;
    __shared__ float vx[G][NP], vu[G][NP], vl[G][NP], vq[G][NP], vr[G][NP];
    const Ix<SH> ix{p.N};
    const int gl = threadIdx.x / NP, i = threadIdx.x % NP, b = blockIdx.y;
    const int k = blockIdx.x * G + gl;
    const bool kv = k < p.N, dyn = k < p.N - 1;
    const int kk = kv ? k : 0;
    // dx_k, du_k and lambda_{k+1}, whole, for every lane of the group
    vx[gl][i] = (kv && i < n) ? p.dz[ix.dx(b, kk, i)] : 0.0f;
    vu[gl][i] = (dyn && i < m) ? p.dz[ix.du(b, kk, i)] : 0.0f;
    vl[gl][i] = (dyn && i < n) ? p.lambda[ix.vn(b, kk + 1, i)] : 0.0f;
    __syncthreads();
    float qv, rv, ev, x0v;
    {
        const bool rowv = kv && i < n;
        const float lam = rowv ? p.lambda[ix.vn(b, kk, i)] : 0.0f;
        const float dxn = (dyn && i < n) ? p.dz[ix.dx(b, kk + 1, i)] : 0.0f;
        kkt_rows<SH>(p, b, kk, i, kv, vx[gl], vu[gl], vl[gl], lam, dxn, qv, rv, ev, x0v);
    }
    if (kv && i < n) {
        if (dyn) ec[ix.e(b, kk, i)] = ev;
        qc[ix.vn(b, kk, i)] = qv;
        if (k == 0) x0c[(size_t)b * n + i] = x0v;
    }
    if (dyn && i < m) rc[ix.vm(b, kk, i)] = rv;
    vq[gl][i] = qv;
    vr[gl][i] = rv;
    __syncthreads();
    // h_k = Q~_k^-1 q'_k and R_k^-1 r'_k, row i
    float h = 0.0f, g = 0.0f;
    if (kv && i < n) {
        const float* Qi = p.Qinv + ix.Q(b, kk, i);
#pragma unroll
        for (int c = 0; c < n; ++c) h = fmaf(Qi[c], vq[gl][c], h);
        hq[ix.vn(b, kk, i)] = h;
    }
    if (dyn && i < m) {
        const float* Ri = p.Rinv + ix.R(b, kk, i);
#pragma unroll
        for (int c = 0; c < m; ++c) g = fmaf(Ri[c], vr[gl][c], g);
    }
    __syncthreads();  // the vectors above are read; their rows take h and R^-1 r'
    vq[gl][i] = h;
    vr[gl][i] = g;
    __syncthreads();
    if (dyn && i < n) {  // t_k = A_k h_k + B_k R_k^-1 r'_k, row i
        const float* Ar = p.A + ix.A(b, kk, i);
        const float* Br = p.Bu + ix.Bu(b, kk, i);
        float t = 0.0f;
#pragma unroll
        for (int c = 0; c < n; ++c) t = fmaf(Ar[c], vq[gl][c], t);
#pragma unroll
        for (int c = 0; c < m; ++c) t = fmaf(Br[c], vr[gl][c], t);
        tq[ix.vn(b, kk, i)] = t;
    }
}

// The correction's gamma from k_kkt_residual's h_k and t_k; one thread per entry.
__global__ void k_refine_gamma(float* gamma, const float* hq, const float* tq, const float* ec, const float* x0c,
                               int n, int N, size_t total)
{
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const size_t b = t / ((size_t)N * n), r = t % ((size_t)N * n);
    const int k = (int)(r / n), i = (int)(r % n);
    gamma[t] = k == 0 ? x0c[b * n + i] + hq[t]
                      : ec[(b * (N - 1) + (k - 1)) * n + i] - tq[t - n] + hq[t];
}

// lambda += the correction's lambda, dz += its dz, flags |= its flags.
__global__ void k_refine_add(float* lam, const float* lamc, size_t nlam, float* dz, const float* dzc, size_t ndz,
                             int32_t* flags, const int32_t* flc, int B)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < nlam + ndz + B; t += stride) {
        if (t < nlam)
            lam[t] += lamc[t];
        else if (t < nlam + ndz)
            dz[t - nlam] += dzc[t - nlam];
        else
            flags[t - nlam - ndz] |= flc[t - nlam - ndz];
    }
}

template <class SH>
struct FormOnlyLds {
    FormLds<SH> f;
    Park<SH> park;
};

// Copy nf floats from LDS to global memory with the threads t = t0, t0 + nt, ...
// of the caller, 16 bytes per access when both ends allow it.
__device__ __forceinline__ void lds_to_global(float* dst, const float* src, int nf, int t0, int nt)
{
    if (nf <= 0) return;
    const bool vec = ((reinterpret_cast<size_t>(dst) | reinterpret_cast<size_t>(src)) & 15) == 0;
    int done = 0;
    if (vec) {
        const int n4 = nf / 4;
        const float4* s4 = reinterpret_cast<const float4*>(src);
        float4* d4 = reinterpret_cast<float4*>(dst);
#pragma unroll 4
        for (int j = t0; j < n4; j += nt) d4[j] = s4[j];
        done = 4 * n4;
    }
    for (int j = done + t0; j < nf; j += nt) dst[j] = src[j];
}

// Stage 1 alone.  The outputs leave through LDS so that every store is a
// contiguous 16-byte write: the parked Q~^-1 / R^-1 blocks are already in the
// output layout, and each wave stages the S (and Phi^-1) block rows of its own
// knots in a private slice before writing them out.
template <class SH, bool PRE>
__global__ __launch_bounds__(SH::THREADS) void k_form(Params p)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC, KPW = SH::KPW;
    constexpr int ROWBLK = 3 * NC * NC;  // one knot's block row
    static_assert((SH::THREADS / 64) * KPW * ROWBLK * sizeof(float) <= sizeof(FormOnlyLds<SH>),
                  "the staging slices must fit in the kernel's LDS");
    __shared__ FormOnlyLds<SH> L;
    const Ix<SH> ix{p.N};
    const int N = p.N;
    const int b = blockIdx.x, w = blockIdx.y;
    int w0, o0, o1;
    if (p.win_own <= 0) {
        w0 = 0;
        o0 = 0;
        o1 = N;
    } else {
        o0 = w * p.win_own;
        o1 = min(o0 + p.win_own, N);
        w0 = max(o0 - 2, 0);  // two knots of halo before, one after
    }
    const int nslot = min(o1 + 1, N) - w0;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP, k = w0 + s;
    const bool own = s < nslot && k >= o0 && k < o1;
    Rows<SH> rw;
    int fl = 0;
    form<SH, PRE>(p, b, w0, nslot, L.f, L.park, rw, fl, [](const float*, const float*) {});
    if (own && i == 0 && fl) atomicOr(p.flags + b, fl);
    if (own && i < NC) p.gamma[ix.vn(b, k, i)] = rw.gam;

    // Q~^-1 and R^-1 of the owned knots (contiguous in the park and in memory)
    const int s0 = o0 - w0, s1 = o1 - w0;
    const int nt = blockDim.x, t0 = threadIdx.x;
    lds_to_global(p.Qinv + ix.Q(b, o0, 0), &L.park.Q[s0][0][0], (s1 - s0) * NC * NC, t0, nt);
    const int r1 = min(o1, N - 1);
    if (r1 > o0) lds_to_global(p.Rinv + ix.R(b, o0, 0), &L.park.R[s0][0][0], (r1 - o0) * MC * MC, t0, nt);
    __syncthreads();

    // S and Phi^-1 block rows through a wave-private slice (LDS accesses of one
    // wave complete in order, so no workgroup barrier is needed between them)
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    float* slice = reinterpret_cast<float*>(&L) + (size_t)wave * KPW * ROWBLK;
    const int sw = s % KPW;                                   // this lane's knot within the wave
    const int ws0 = max(s0, wave * KPW), ws1 = min(s1, (wave + 1) * KPW);  // owned slots of the wave
    auto put = [&](float* dst, const float* lo, const float* dg, const float* hi) {
        if (i < NC)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                slice[(sw * 3 + 0) * NC * NC + i * NC + c] = lo[c];
                slice[(sw * 3 + 1) * NC * NC + i * NC + c] = dg[c];
                slice[(sw * 3 + 2) * NC * NC + i * NC + c] = hi[c];
            }
        __builtin_amdgcn_wave_barrier();
        if (ws1 > ws0)
            lds_to_global(dst + ix.blk(b, w0 + ws0, 0, 0), slice + (ws0 - wave * KPW) * ROWBLK, (ws1 - ws0) * ROWBLK,
                          lane, 64);
        __builtin_amdgcn_wave_barrier();
    };
    // S's diagonal and upper blocks, knot by knot (the lower blocks are not read)
    auto put_upper = [&](float* dst, const float* dg, const float* hi) {
        if (i < NC)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                slice[(sw * 3 + 1) * NC * NC + i * NC + c] = dg[c];
                slice[(sw * 3 + 2) * NC * NC + i * NC + c] = hi[c];
            }
        __builtin_amdgcn_wave_barrier();
        for (int ws = ws0; ws < ws1; ++ws)
            lds_to_global(dst + ix.blk(b, w0 + ws, 1, 0), slice + (ws - wave * KPW) * ROWBLK + NC * NC, 2 * NC * NC,
                          lane, 64);
        __builtin_amdgcn_wave_barrier();
    };
    if (!PRE && p.s_upper_only)
        put_upper(p.S, rw.sd, rw.sup);
    else
        put(p.S, rw.slo, rw.sd, rw.sup);
    if constexpr (PRE) put(p.Pinv, rw.plo, rw.pd, rw.pup);
}

// ------------------------------------------------------------------ stage 2 alone

template <class SH, int C, class MAT>
__device__ __forceinline__ void pcg_and_recover(const Params& p, const MAT& M, PcgLds<SH, C>& L, const float* gam,
                                                float* lam)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC, SL = SH::SLOTS;
    const Ix<SH> ix{p.N};
    const int b = blockIdx.x;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    int it = 0, pfl = 0;
    float rel = 0.0f;
    pcg_robust<SH, C>(p, M, gam, lam, L, it, rel, pfl);
#pragma unroll
    for (int c = 0; c < C; ++c) L.xv[c * SL + s + 1][i] = lam[c];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int k = c * SL + s;
        const float lamn = L.xv[k + 2][i];
        const bool kv = k < p.N, hn = kv && k < p.N - 1, rowv = kv && i < NC;
        const bool urow = hn && i < MC;
        float qi[NC], ri[MC], bc[NC], sup[NC];
        ld_row<NC>(p.Qinv, ix.Q(b, k, i), rowv, qi);
        ld_row<MC>(p.Rinv, ix.R(b, k, i), urow, ri);
        ld_row<NC, MC>(p.Bu, ix.Bu(b, k, 0) + i, urow, bc);  // column i of B_k
        M.sup(k, sup);
        const float qv = ld1(p.q, ix.vn(b, k, i), rowv);
        const float rv = ld1(p.r, ix.vm(b, k, i), urow);
        float h = 0.0f;  // (Q~_k^-1 q_k)_i, with the formation's arithmetic
        dotb<NP, NC>(h, Bc<NP>(qv), qi);
        float dx, du;
        recover<SH>(i, rowv, urow, lam[c], lamn, qi, sup, h, bc, rv, ri, dx, du);
        if (rowv) {
            p.lambda[ix.vn(b, k, i)] = lam[c];
            p.dz[ix.dx(b, k, i)] = dx;
        }
        if (hn && i < MC) p.dz[ix.du(b, k, i)] = du;
    }
    if (threadIdx.x == 0) {
        p.iters[b] = it;
        p.relres[b] = rel;
        if (pfl) p.flags[b] |= pfl;
    }
}

template <class SH>
__global__ __launch_bounds__(SH::THREADS) void k_pcg_res(Params p)
{
    constexpr int NP = SH::NP, NC = SH::NC;
    __shared__ PcgLds<SH, 1> L;
    const Ix<SH> ix{p.N};
    const int b = blockIdx.x;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP, k = s;
    const bool rowv = k < p.N && i < NC;
    Rows<SH> rw;
    ld_row<NC>(p.S, ix.blk(b, k, 0, i), rowv, rw.slo);
    ld_row<NC>(p.S, ix.blk(b, k, 1, i), rowv, rw.sd);
    ld_row<NC>(p.S, ix.blk(b, k, 2, i), rowv, rw.sup);
    ld_row<NC>(p.Pinv, ix.blk(b, k, 0, i), rowv, rw.plo);
    ld_row<NC>(p.Pinv, ix.blk(b, k, 1, i), rowv, rw.pd);
    ld_row<NC>(p.Pinv, ix.blk(b, k, 2, i), rowv, rw.pup);
    rw.gam = ld1(p.gamma, ix.vn(b, k, i), rowv);
    float lam = ld1(p.lambda, ix.vn(b, k, i), rowv);
    const RegMat<SH> M{&rw};
    pcg_and_recover<SH, 1>(p, M, L, &rw.gam, &lam);
}

template <class SH, int C>
__global__ __launch_bounds__(SH::THREADS) void k_pcg_stream(Params p)
{
    constexpr int NP = SH::NP, SL = SH::SLOTS, NC = SH::NC;
    __shared__ PcgLds<SH, C> L;
    const Ix<SH> ix{p.N};
    const int b = blockIdx.x;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    float gam[C], lam[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int k = c * SL + s;
        const bool rowv = k < p.N && i < NC;
        gam[c] = ld1(p.gamma, ix.vn(b, k, i), rowv);
        lam[c] = ld1(p.lambda, ix.vn(b, k, i), rowv);
    }
    if constexpr (C == 2 && NP == 16) {
        // two knots per lane group: S's diagonal rows in registers and the D_k^-1 in
        // LDS (HybMat), so only S's off-diagonal blocks stream at every iteration
        constexpr int DS = NC | 1;  // odd row stride: a lane group's rows fall in distinct banks
        __shared__ float dinv[2 * SL][NC][DS];
        float sd[C][NC];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int k = c * SL + s;
            const bool rowv = k < p.N && i < NC;
            float t[NC];
            ld_row<NC>(p.S, ix.blk(b, k, 1, i), rowv, sd[c]);
            ld_row<NC>(p.Pinv, ix.blk(b, k, 1, i), rowv, t);
            if (i < NC)
#pragma unroll
                for (int col = 0; col < NC; ++col) dinv[k][i][col] = t[col];
        }
        __syncthreads();
        const HybMat<SH, C, DS> M{p.S, ix, b, i, sd, dinv, L.xy};
        pcg_and_recover<SH, C>(p, M, L, gam, lam);
    } else {
        // phased for 16-lane groups (less traffic); 32-lane ones measure faster without the extra barrier
        const GlobalMat<SH, NP == 16> M{p.S, p.Pinv, ix, b, i, L.xy};
        pcg_and_recover<SH, C>(p, M, L, gam, lam);
    }
}

// ------------------------------------------------------------------ stage 2, direct

// One 64-lane workgroup, one solve per lane group (64 / NP solves): the
// elimination walks the knots in order, so the solves of a wave move in step.
template <class SH>
__global__ __launch_bounds__(64) void k_direct(Params p)
{
    constexpr int SPW = 64 / SH::NP;
    __shared__ __align__(16) float piv[SPW][GJ_LDS_BLOCK * ((SH::NC + 3) / 4 * 4)];  // pivot rows (32-lane groups)
    const int b = blockIdx.x * SPW + (int)(threadIdx.x / SH::NP);
    direct_solve<SH>(p, b, b < p.B, piv[threadIdx.x / SH::NP]);
}

// ------------------------------------------------------------------ stage 3 alone

template <class SH, int LPL>
__global__ __launch_bounds__(1024) void k_merit(Params p)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC, P = 16 * LPL;
    __shared__ __align__(16) float mer[(GATO_MAX_ALPHA + 1) * P];
    const Ix<SH> ix{p.N};
    const int b = blockIdx.x;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    const int ks = blockDim.x / NP;
    for (int t = threadIdx.x; t < (p.n_alpha + 1) * P; t += blockDim.x) mer[t] = 0.0f;
    __syncthreads();
    for (int c0 = 0; c0 < p.N; c0 += ks) {
        const int k = c0 + s;
        const bool kv = k < p.N, hn = kv && k < p.N - 1, rowv = kv && i < NC;
        const float dx = ld1(p.dz, ix.dx(b, k, i), rowv);
        const float du = ld1(p.dz, ix.du(b, k, i), hn && i < MC);
        const float dxn = ld1(p.dz, ix.dx(b, k + 1, i), hn && i < NC);
        MeritIn<SH> mi;
        wave_prio<true, 3>();
        merit_rows<SH>(p, b, k, i, mi);
        wave_prio<true, 2>();
        merit_knot<SH>(p, k, i, mi, dx, du, dxn, mer + (kv ? k : 0), P);
    }
    wave_prio<true, 0>();
    __syncthreads();
    int32_t best;
    int lsfail;
    merit_select<LPL>(p, b, mer, P, best, lsfail);
    if (threadIdx.x == 0) {
        p.best[b] = best;
        if (lsfail) p.flags[b] |= GATO_F_LS_FAILED;
    }
}

// The per-knot merit values of one solve spread over gridDim.y workgroups
// (knots y N / Y .. (y + 1) N / Y - 1 in workgroup y), into p.mpart, for
// batches too small to fill the device with one workgroup per solve; then
// k_merit_sum forms the same canonical sums as k_merit, so the bits match.
template <class SH>
__global__ __launch_bounds__(1024) void k_merit_knots(Params p)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC;
    const Ix<SH> ix{p.N};
    const int b = blockIdx.x;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    const int ks = blockDim.x / NP;
    const int k0 = (int)((long long)blockIdx.y * p.N / gridDim.y);
    const int k1 = (int)((long long)(blockIdx.y + 1) * p.N / gridDim.y);
    float* out = p.mpart + (size_t)b * (p.n_alpha + 1) * p.N;
    for (int c0 = k0; c0 < k1; c0 += ks) {
        const int k = c0 + s < k1 ? c0 + s : p.N;  // p.N: no knot (loads masked, nothing written)
        const bool kv = k < p.N, hn = kv && k < p.N - 1, rowv = kv && i < NC;
        const float dx = ld1(p.dz, ix.dx(b, k, i), rowv);
        const float du = ld1(p.dz, ix.du(b, k, i), hn && i < MC);
        const float dxn = ld1(p.dz, ix.dx(b, k + 1, i), hn && i < NC);
        MeritIn<SH> mi;
        merit_rows<SH>(p, b, k, i, mi);
        merit_knot<SH>(p, k, i, mi, dx, du, dxn, out + (kv ? k : 0), p.N);
    }
}

template <int LPL>
__global__ __launch_bounds__(256) void k_merit_sum(Params p)
{
    constexpr int P = 16 * LPL;
    __shared__ __align__(16) float mer[(GATO_MAX_ALPHA + 1) * P];
    const int b = blockIdx.x;
    const float* in = p.mpart + (size_t)b * (p.n_alpha + 1) * p.N;
    // row j of the values, zero-padded to P leaves; eight loads in flight per thread
    const int tot = (p.n_alpha + 1) * P;
    for (int t0 = threadIdx.x; t0 < tot; t0 += 8 * blockDim.x) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int t = t0 + u * blockDim.x, j = t / P, k = t % P;
            v[u] = (t < tot && k < p.N) ? in[(size_t)j * p.N + k] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (t0 + u * blockDim.x < tot) mer[t0 + u * blockDim.x] = v[u];
    }
    __syncthreads();
    int32_t best;
    int lsfail;
    if (merit_select<LPL>(p, b, mer, P, best, lsfail) && threadIdx.x == 0) {
        p.best[b] = best;
        if (lsfail) p.flags[b] |= GATO_F_LS_FAILED;
    }
}

// Candidate-parallel variant: one workgroup per (solve, step size), each
// recomputing a knot's step-size-independent products for its own step size
// (the pages' per-candidate launch, against the fused per-knot evaluation of
// k_merit).  A knot's value comes from the same arithmetic as in k_merit and
// the sum over knots from the same pairwise tree, so both give identical bits.
template <class SH, int LPL>
__global__ __launch_bounds__(1024) void k_merit_cand(Params p)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC, P = 16 * LPL;
    __shared__ __align__(16) float mer[P];
    const Ix<SH> ix{p.N};
    const int b = blockIdx.x, j = blockIdx.y;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    const int ks = blockDim.x / NP;
    for (int t = threadIdx.x; t < P; t += blockDim.x) mer[t] = 0.0f;
    __syncthreads();
    for (int c0 = 0; c0 < p.N; c0 += ks) {
        const int k = c0 + s;
        const bool kv = k < p.N, hn = kv && k < p.N - 1, rowv = kv && i < NC;
        const float dx = ld1(p.dz, ix.dx(b, k, i), rowv);
        const float du = ld1(p.dz, ix.du(b, k, i), hn && i < MC);
        const float dxn = ld1(p.dz, ix.dx(b, k + 1, i), hn && i < NC);
        MeritIn<SH> mi;
        merit_rows<SH>(p, b, k, i, mi);
        const MeritPrep m = merit_prep<SH>(p, k, mi, dx, du, dxn);
        const float v = merit_value<SH>(p, k, mi, m, dx, j);
        if (i == 0 && kv) mer[k] = v;
    }
    __syncthreads();
    if (threadIdx.x >= 64) return;
    const float tot = canon_sum<LPL>(mer);
    if (threadIdx.x == 0) {
        if (j == 0)
            p.merit0[b] = tot;
        else
            p.merit[(size_t)b * p.n_alpha + (j - 1)] = tot;
    }
}

// Selection after k_merit_cand (the rule of merit_select), one thread per solve.
__global__ void k_merit_pick(Params p)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= p.B) return;
    const float M0 = p.merit0[b];
    float bv = 0.0f;
    int bi = 0;
    for (int j = 1; j <= p.n_alpha; ++j) {
        const float v = p.merit[(size_t)b * p.n_alpha + (j - 1)];
        if (j == 1 || v < bv) {
            bv = v;
            bi = j - 1;
        }
    }
    const bool lsfail = !(bv < M0);
    p.best[b] = lsfail ? -1 : bi;
    if (lsfail) p.flags[b] |= GATO_F_LS_FAILED;
}

// ------------------------------------------------------------------ host side

// Workgroup size of the standalone merit: enough waves for every knot at once,
// at most 16 (waves = 0), or the caller's choice.
static int merit_waves(int N, int kpw, int waves)
{
    if (waves >= 1 && waves <= 16) return waves;
    int w = (N + kpw - 1) / kpw;
    return w < 1 ? 1 : (w > 16 ? 16 : w);
}

template <class SH>
struct Ops {
    static constexpr int SL = SH::SLOTS, KPW = SH::KPW;
    static int threads_for(int knots) { return ((knots + KPW - 1) / KPW) * 64; }
    static bool fused_ok(int N) { return N <= SL; }
    static int stream_chunks(int N) { return N <= SL ? 1 : (N <= 2 * SL ? 2 : (N <= 4 * SL ? 4 : 0)); }

    // Horizons longer than a workgroup are formed in windows.  For n <= 16 the
    // windows hold 32 knots (512 threads, half the LDS), so that two workgroups
    // share a CU and one's loads and stores overlap the other's arithmetic.
    using WinShape = Shape<SH::NC, SH::MC, SH::NP == 16 ? SH::SLOTS / 2 : SH::SLOTS>;
    template <class FS>
    static void form_launch(const Params& q, int nwin, int threads, hipStream_t st, bool pre)
    {
        if (pre)
            hipLaunchKernelGGL((k_form<FS, true>), dim3(q.B, nwin), dim3(threads), 0, st, q);
        else
            hipLaunchKernelGGL((k_form<FS, false>), dim3(q.B, nwin), dim3(threads), 0, st, q);
    }
    static hipError_t form(const Params& p, hipStream_t st, bool pre = true)
    {
        Params q = p;
        hipLaunchKernelGGL(k_zero_i32, dim3((p.B + 255) / 256), dim3(256), 0, st, p.flags, p.B);
        if (p.N <= SL) {
            q.win_own = 0;
            form_launch<SH>(q, 1, threads_for(p.N), st, pre);
        } else {
            q.win_own = WinShape::SLOTS - 3;
            form_launch<WinShape>(q, (p.N + q.win_own - 1) / q.win_own, WinShape::THREADS, st, pre);
        }
        return hipGetLastError();
    }
    static hipError_t pcg(const Params& p, hipStream_t st)
    {
        const int C = stream_chunks(p.N);
        if (C == 1) {
            hipLaunchKernelGGL((k_pcg_res<SH>), dim3(p.B), dim3(threads_for(p.N)), 0, st, p);
        } else if (C == 2) {
            hipLaunchKernelGGL((k_pcg_stream<SH, 2>), dim3(p.B), dim3(SH::THREADS), 0, st, p);
        } else if (C == 4) {
            hipLaunchKernelGGL((k_pcg_stream<SH, 4>), dim3(p.B), dim3(SH::THREADS), 0, st, p);
        } else {
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    static hipError_t merit(const Params& p, hipStream_t st, int variant = GATO_MERIT_PER_KNOT, int waves = 0)
    {
        const int P = leaves_for(p.N);
        const dim3 blk(merit_waves(p.N, KPW, waves) * 64);
        if (variant == GATO_MERIT_PER_CANDIDATE) {
            const dim3 g(p.B, p.n_alpha + 1);
            switch (P / 16) {
                case 4: hipLaunchKernelGGL((k_merit_cand<SH, 4>), g, blk, 0, st, p); break;
                case 8: hipLaunchKernelGGL((k_merit_cand<SH, 8>), g, blk, 0, st, p); break;
                case 16: hipLaunchKernelGGL((k_merit_cand<SH, 16>), g, blk, 0, st, p); break;
                case 32: hipLaunchKernelGGL((k_merit_cand<SH, 32>), g, blk, 0, st, p); break;
                case 64: hipLaunchKernelGGL((k_merit_cand<SH, 64>), g, blk, 0, st, p); break;
                default: return hipErrorInvalidValue;
            }
            hipLaunchKernelGGL(k_merit_pick, dim3((p.B + 255) / 256), dim3(256), 0, st, p);
            return hipGetLastError();
        }
        const dim3 g(p.B);
        switch (P / 16) {
            case 4: hipLaunchKernelGGL((k_merit<SH, 4>), g, blk, 0, st, p); break;
            case 8: hipLaunchKernelGGL((k_merit<SH, 8>), g, blk, 0, st, p); break;
            case 16: hipLaunchKernelGGL((k_merit<SH, 16>), g, blk, 0, st, p); break;
            case 32: hipLaunchKernelGGL((k_merit<SH, 32>), g, blk, 0, st, p); break;
            case 64: hipLaunchKernelGGL((k_merit<SH, 64>), g, blk, 0, st, p); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    // gato_sqp_step's merit with a workspace: a solve's knots spread over
    // several workgroups when one workgroup per solve would leave the device
    // short of work (512 workgroups wanted: two resident per CU, no second
    // round), each taking at least one pass of 1024 / NP knots; else the
    // one-kernel form.
    static int merit_split(const Params& p)
    {
        const int per_pass = 1024 / SH::NP;
        const int by_knots = (p.N + per_pass - 1) / per_pass;
        const int by_batch = 512 / p.B;
        return std::max(1, std::min(by_knots, by_batch));
    }
    static hipError_t merit_ws(const Params& p, hipStream_t st)
    {
        const int y = merit_split(p);
        if (y == 1 || p.mpart == nullptr) return merit(p, st);
        hipLaunchKernelGGL((k_merit_knots<SH>), dim3(p.B, y), dim3(1024), 0, st, p);
        switch (leaves_for(p.N) / 16) {
            case 4: hipLaunchKernelGGL((k_merit_sum<4>), dim3(p.B), dim3(256), 0, st, p); break;
            case 8: hipLaunchKernelGGL((k_merit_sum<8>), dim3(p.B), dim3(256), 0, st, p); break;
            case 16: hipLaunchKernelGGL((k_merit_sum<16>), dim3(p.B), dim3(256), 0, st, p); break;
            case 32: hipLaunchKernelGGL((k_merit_sum<32>), dim3(p.B), dim3(256), 0, st, p); break;
            case 64: hipLaunchKernelGGL((k_merit_sum<64>), dim3(p.B), dim3(256), 0, st, p); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    static hipError_t residual(const Params& p, float* qc, float* rc, float* ec, float* x0c, float* hq, float* tq,
                               hipStream_t st)
    {
        constexpr int G = 256 / SH::NP;
        hipLaunchKernelGGL((k_kkt_residual<SH>), dim3((p.N + G - 1) / G, p.B), dim3(256), 0, st, p, qc, rc, ec, x0c,
                           hq, tq);
        return hipGetLastError();
    }
    static hipError_t direct(const Params& p, hipStream_t st)
    {
        constexpr int SPW = 64 / SH::NP;
        hipLaunchKernelGGL((k_direct<SH>), dim3((p.B + SPW - 1) / SPW), dim3(64), 0, st, p);
        return hipGetLastError();
    }
    // The PCG's stop test on the vector unit at up to two waves per SIMD (pcg())
    static hipError_t fused(const Params& p, hipStream_t st)
    {
        const int threads = threads_for(p.N);
        if constexpr (SH::THREADS <= 512) {
            hipLaunchKernelGGL((k_sqp_fused<SH, true>), dim3(p.B), dim3(threads), 0, st, p);
        } else {
            if (threads <= 512)
                hipLaunchKernelGGL((k_sqp_fused<SH, true>), dim3(p.B), dim3(threads), 0, st, p);
            else
                hipLaunchKernelGGL((k_sqp_fused<SH, false>), dim3(p.B), dim3(threads), 0, st, p);
        }
        return hipGetLastError();
    }
    // formation (windowed), the direct solve and the merit take any N up to the
    // merit's 1024 leaves; PCG holds at most four knots per lane group
    static bool supported(int N) { return N >= 1 && leaves_for(N) <= 1024; }
    static bool pcg_supported(int N) { return N >= 1 && stream_chunks(N) != 0; }
};

// Shapes the library has kernels for (GATO_FOR_SHAPES).
template <class F>
static int with_shape(int n, int m, F&& f)
{
#define GATO_SHAPE(n_, m_) \
    if (n == n_ && m == m_) return f(Ops<Shape<n_, m_>>{});
    GATO_FOR_SHAPES(GATO_SHAPE)
#undef GATO_SHAPE
    return GATO_E_UNSUPPORTED;
}

static bool aligned4(const void* ptr) { return ((uintptr_t)ptr & 3u) == 0; }

static int check_ptrs(std::initializer_list<const void*> req)
{
    for (const void* x : req)
        if (x == nullptr) return GATO_E_NULL;
    for (const void* x : req)
        if (!aligned4(x)) return GATO_E_ALIGN;
    return GATO_OK;
}

// Dims of a shape the library has kernels for (every entry point).
static int check_dims(const gato_dims_t* d)
{
    if (d == nullptr) return GATO_E_NULL;
    if (d->n < 1 || d->m < 1 || d->N < 1 || d->B < 0) return GATO_E_DIMS;
    if (gato_shape_supported(d->n, d->m, d->N) != 1) return GATO_E_UNSUPPORTED;
    return GATO_OK;
}

// Dims gato_sqp_step serves: a shape with kernels, or one it embeds in a larger
// shape that has them (padded_dims).
static int check_dims_step(const gato_dims_t* d)
{
    if (d == nullptr) return GATO_E_NULL;
    if (d->n < 1 || d->m < 1 || d->N < 1 || d->B < 0) return GATO_E_DIMS;
    if (gato_shape_supported(d->n, d->m, d->N) == 0) return GATO_E_UNSUPPORTED;
    return GATO_OK;
}

// Arrays indexed by the dynamics (R, r, A, Bu, e, Rinv) are empty when N = 1.
static const void* dyn(const void* x, const gato_dims_t* d)
{
    static const int dummy = 0;
    return (d->N == 1 && x == nullptr) ? &dummy : x;
}

static Params make_params(const gato_dims_t* d)
{
    Params p;
    std::memset(&p, 0, sizeof(p));
    p.n = d->n;
    p.m = d->m;
    p.N = d->N;
    p.B = d->B;
    return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// gato_sqp_step's workspace beyond the fused horizons.  Only the direct solves
// run there, so it holds no Phi^-1.
struct WsLayout {
    size_t S, mpart, gamma, Qinv, Rinv, direct, qc, rc, ec, x0c, hq, tq, lamc, dzc, flc, total;
};

static size_t direct_ws_bytes(const gato_dims_t* d)
{
    const size_t B = d->B, N = d->N, n = d->n;
    return align256(B * N * n * (n + 1) * sizeof(float));
}

static WsLayout ws_layout(const gato_dims_t* d)
{
    const size_t B = d->B, N = d->N, n = d->n, m = d->m;
    WsLayout w;
    size_t off = 0;
    w.S = off;
    off += align256(B * N * 3 * n * n * sizeof(float));
    w.mpart = off;  // the merit's per-knot values
    off += align256(B * (GATO_MAX_ALPHA + 1) * N * sizeof(float));
    w.gamma = off;
    off += align256(B * N * n * sizeof(float));
    w.Qinv = off;
    off += align256(B * N * n * n * sizeof(float));
    w.Rinv = off;
    off += align256(B * (N > 1 ? N - 1 : 1) * m * m * sizeof(float));
    w.direct = off;  // the block Thomas or the cyclic-reduction solve's workspace
    off += std::max(direct_ws_bytes(d), cr_ws_bytes(d));
    // the refinement pass: the correction system's q, r, e, x0, the terms of its gamma
    // (h_k, t_k) and its lambda, dz, flags
    const size_t Nd = N > 1 ? N - 1 : 0;
    w.qc = off;
    off += align256(B * N * n * sizeof(float));
    w.rc = off;
    off += align256(B * Nd * m * sizeof(float));
    w.ec = off;
    off += align256(B * Nd * n * sizeof(float));
    w.x0c = off;
    off += align256(B * n * sizeof(float));
    w.hq = off;
    off += align256(B * N * n * sizeof(float));
    w.tq = off;
    off += align256(B * N * n * sizeof(float));
    w.lamc = off;
    off += align256(B * N * n * sizeof(float));
    w.dzc = off;
    off += align256(B * (N * n + Nd * m) * sizeof(float));
    w.flc = off;
    off += align256(B * sizeof(int32_t));
    w.total = off;
    return w;
}

static bool fused_path(const gato_dims_t* d)
{
    return with_shape(d->n, d->m, [&](auto ops) { return decltype(ops)::fused_ok(d->N) ? 1 : 0; }) == 1;
}

// ------------------------------------------------------------------ shapes served by padding

// A problem of a shape without kernels of its own is solved inside the smallest
// shape with kernels that holds it (fewest states, then fewest controls): its
// Q_k and R_k get identity rows and columns beyond n and m, A_k, B_k, q, r, e
// and x0 zeros.  The added states then have x0 = 0, e = 0 and no coupling to the
// others, and the added controls no effect on any state, so the padded QP is the
// original one plus a separate part whose solution is zero: its dz and lambda
// entries are exactly zero (PCG keeps them at zero from a zero start, since the
// padded blocks of S and Phi^-1 do not couple them to the rest), and its merit
// terms are zero.  The original problem's dz, lambda, merits and flags are the
// padded problem's, read at the original rows.
static bool native_shape(int n, int m)
{
    return with_shape(n, m, [](auto) { return 1; }) == 1;
}

static bool padded_dims(const gato_dims_t* d, gato_dims_t* pd)
{
    int bn = 0, bm = 0;
#define GATO_PAD_SHAPE(n_, m_) \
    if (n_ >= d->n && m_ >= d->m && (bn == 0 || n_ < bn || (n_ == bn && m_ < bm))) { bn = n_; bm = m_; }
    GATO_FOR_SHAPES(GATO_PAD_SHAPE)
#undef GATO_PAD_SHAPE
    if (bn == 0) return false;
    *pd = *d;
    pd->n = bn;
    pd->m = bm;
    return true;
}

// The padded copies in gato_sqp_step's workspace, then the padded step's own workspace.
struct PadLayout {
    size_t Q, q, R, r, A, Bu, e, x0, lam, dz, inner, total;
};

// direct: the inner call runs a direct solve even where the fused path applies
// (an explicit solver in gato_step_opts_t).
static PadLayout pad_layout(const gato_dims_t* pd, bool direct)
{
    const size_t B = pd->B, N = pd->N, n = pd->n, m = pd->m, Nd = N > 1 ? N - 1 : 0;
    PadLayout w;
    size_t off = 0;
    auto take = [&](size_t floats) {
        const size_t at = off;
        off += align256(floats * sizeof(float));
        return at;
    };
    w.Q = take(B * N * n * n);
    w.q = take(B * N * n);
    w.R = take(B * Nd * m * m);
    w.r = take(B * Nd * m);
    w.A = take(B * Nd * n * n);
    w.Bu = take(B * Nd * n * m);
    w.e = take(B * Nd * n);
    w.x0 = take(B * n);
    w.lam = take(B * N * n);
    w.dz = take(B * (N * n + Nd * m));
    w.inner = off;
    w.total = off + ((fused_path(pd) && !direct) ? 0 : ws_layout(pd).total);
    return w;
}

// dst: nblk blocks of Rp x Cp from src's nblk blocks of R x C (R <= Rp, C <= Cp):
// the source entry where there is one, else `diag` on the diagonal and 0 off it.
__global__ void k_pad_blocks(float* dst, const float* src, size_t nblk, int R, int C, int Rp, int Cp, float diag)
{
    const size_t per = (size_t)Rp * Cp, total = nblk * per;
    for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
        const size_t blk = t / per;
        const int r = (int)((t % per) / Cp), c = (int)(t % Cp);
        dst[t] = (r < R && c < C) ? src[(blk * R + r) * C + c] : (r == c ? diag : 0.0f);
    }
}

// The inverse: dst's nblk blocks of R x C from the leading rows and columns of src's Rp x Cp blocks.
__global__ void k_unpad_blocks(float* dst, const float* src, size_t nblk, int R, int C, int Rp, int Cp)
{
    const size_t per = (size_t)R * C, total = nblk * per;
    for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
        const size_t blk = t / per;
        const int r = (int)((t % per) / C), c = (int)(t % C);
        dst[t] = src[(blk * Rp + r) * Cp + c];
    }
}

// dz [B][N n + (N-1) m] (dx_0, du_0, ..., dx_{N-1}) from the padded step's [B][N np + (N-1) mp].
__global__ void k_unpad_dz(float* dz, const float* dzp, int B, int N, int n, int m, int np, int mp)
{
    const size_t per = (size_t)N * n + (size_t)(N - 1) * m, perp = (size_t)N * np + (size_t)(N - 1) * mp;
    const size_t total = (size_t)B * per;
    for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
        const size_t b = t / per, o = t % per;
        const size_t k = o / (size_t)(n + m);
        const int w = (int)(o % (size_t)(n + m));  // the last knot has w < n only
        dz[t] = dzp[b * perp + k * (size_t)(np + mp) + (w < n ? w : np + (w - n))];
    }
}

static hipError_t pad_launch(hipStream_t st, float* dst, const float* src, size_t nblk, int R, int C, int Rp, int Cp,
                             float diag)
{
    const size_t total = nblk * (size_t)Rp * Cp;
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_pad_blocks, dim3(grid), dim3(256), 0, st, dst, src, nblk, R, C, Rp, Cp, diag);
    return hipGetLastError();
}

static hipError_t unpad_launch(hipStream_t st, float* dst, const float* src, size_t nblk, int R, int C, int Rp, int Cp)
{
    const size_t total = nblk * (size_t)R * C;
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_unpad_blocks, dim3(grid), dim3(256), 0, st, dst, src, nblk, R, C, Rp, Cp);
    return hipGetLastError();
}

// ------------------------------------------------------------------ allocation-free scratch

// gato_sqp_step_noalloc's workspace: one array per device, held from the load of
// this code object on that device until the process ends.  Host code never
// uses its name as an address (on the host it is a stand-in, not device
// memory); the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[GATO_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the calling thread's current device, looked
// up on the first call there (with that device current); nullptr if the lookup
// fails.
static void* scratch_ptr()
{
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

}  // namespace gato

using namespace gato;

extern "C" {

int gato_shape_supported(int32_t n, int32_t m, int32_t N)
{
    if (n < 1 || m < 1 || N < 1) return 0;
    if (native_shape(n, m)) return with_shape(n, m, [&](auto ops) { return decltype(ops)::supported(N) ? 1 : 0; });
    gato_dims_t d{n, m, N, 1}, pd;
    if (!padded_dims(&d, &pd)) return 0;
    return with_shape(pd.n, pd.m, [&](auto ops) { return decltype(ops)::supported(N) ? 2 : 0; });
}

const char* gato_status_string(int code)
{
    switch (code) {
        case GATO_OK: return "ok";
        case GATO_E_NULL: return "a required pointer is NULL";
        case GATO_E_DIMS: return "dimensions out of range";
        case GATO_E_ALIGN: return "a pointer is not 4-byte aligned";
        case GATO_E_PARAM: return "a scalar parameter is out of range";
        case GATO_E_HIP: return "a HIP launch failed";
        case GATO_E_UNSUPPORTED: return "no kernel for this (n, m, N) in this build";
        case GATO_E_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status code";
    }
}

int gato_step_solver(const gato_dims_t* dims)
{
    const int rc = check_dims_step(dims);
    if (rc) return rc;
    gato_dims_t d = *dims;
    if (!native_shape(d.n, d.m)) padded_dims(dims, &d);
    if (fused_path(&d)) return GATO_SOLVER_FUSED_PCG;
    return cr_preferred(&d, true) ? GATO_SOLVER_CR : GATO_SOLVER_THOMAS;
}

size_t gato_workspace_bytes(const gato_dims_t* dims, int32_t n_alpha)
{
    (void)n_alpha;
    if (check_dims_step(dims) != GATO_OK || dims->B == 0) return 0;
    if (!native_shape(dims->n, dims->m)) {
        gato_dims_t pd;
        padded_dims(dims, &pd);
        return pad_layout(&pd, false).total;
    }
    if (fused_path(dims)) return 0;
    return ws_layout(dims).total;
}

size_t gato_step_workspace_bytes(const gato_dims_t* dims, int32_t n_alpha, const gato_step_opts_t* opts)
{
    if (opts && ((opts->solver != GATO_SOLVER_AUTO && opts->solver != GATO_SOLVER_THOMAS &&
                  opts->solver != GATO_SOLVER_CR && opts->solver != GATO_SOLVER_CR_STREAM) ||
                 (opts->refine != 0 && opts->refine != 1)))
        return 0;  // choices gato_sqp_step_opts rejects
    if (opts == nullptr || opts->solver == GATO_SOLVER_AUTO) return gato_workspace_bytes(dims, n_alpha);
    if (check_dims_step(dims) != GATO_OK || dims->B == 0) return 0;
    if (!native_shape(dims->n, dims->m)) {
        gato_dims_t pd;
        padded_dims(dims, &pd);
        return pad_layout(&pd, true).total;
    }
    return ws_layout(dims).total;
}

int gato_form_schur(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                    const float* r, const float* A, const float* Bu, const float* e,
                    const float* x0, const float* rho, float* S, float* Pinv, float* gamma,
                    float* Qinv, float* Rinv, int32_t* flags, hipStream_t stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->B == 0) return GATO_OK;  // nothing to do; pointers may be empty
    rc = check_ptrs({Q, q, dyn(R, dims), dyn(r, dims), dyn(A, dims), dyn(Bu, dims), dyn(e, dims), x0, S,
                     Pinv, gamma, Qinv, dyn(Rinv, dims), flags});
    if (rc) return rc;
    if (rho && !aligned4(rho)) return GATO_E_ALIGN;
    Params p = make_params(dims);
    p.Q = Q; p.q = q; p.R = R; p.r = r; p.A = A; p.Bu = Bu; p.e = e; p.x0 = x0; p.rho = rho;
    p.S = S; p.Pinv = Pinv; p.gamma = gamma; p.Qinv = Qinv; p.Rinv = Rinv; p.flags = flags;
    return with_shape(dims->n, dims->m, [&](auto ops) {
        return decltype(ops)::form(p, stream) == hipSuccess ? GATO_OK : GATO_E_HIP;
    });
}

int gato_pcg_solve(const gato_dims_t* dims, const float* S, const float* Pinv,
                   const float* gamma, const float* Qinv, const float* Rinv, const float* A,
                   const float* Bu, const float* q, const float* r, float eps, int32_t max_iters,
                   float* lambda, float* dz, int32_t* iters, float* relres, int32_t* flags,
                   hipStream_t stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->B == 0) return GATO_OK;  // nothing to do; pointers may be empty
    rc = check_ptrs({S, Pinv, gamma, Qinv, dyn(Rinv, dims), dyn(Bu, dims), q, dyn(r, dims),
                     lambda, dz, iters, relres, flags});
    if (rc) return rc;
    if (A && !aligned4(A)) return GATO_E_ALIGN;  // not read: the recovery takes A_k' from S_{k,k+1}
    if (!(eps > 0.0f) || max_iters < 1) return GATO_E_PARAM;
    if (with_shape(dims->n, dims->m, [&](auto ops) { return decltype(ops)::pcg_supported(dims->N) ? 1 : 0; }) != 1)
        return GATO_E_UNSUPPORTED;
    Params p = make_params(dims);
    p.S = const_cast<float*>(S); p.Pinv = const_cast<float*>(Pinv); p.gamma = const_cast<float*>(gamma);
    p.Qinv = const_cast<float*>(Qinv); p.Rinv = const_cast<float*>(Rinv);
    p.Bu = Bu; p.q = q; p.r = r;
    p.eps = eps; p.max_iters = max_iters;
    p.lambda = lambda; p.dz = dz; p.iters = iters; p.relres = relres; p.flags = flags;
    return with_shape(dims->n, dims->m, [&](auto ops) {
        return decltype(ops)::pcg(p, stream) == hipSuccess ? GATO_OK : GATO_E_HIP;
    });
}

size_t gato_direct_workspace_bytes(const gato_dims_t* dims)
{
    if (check_dims(dims) != GATO_OK || dims->B == 0) return 0;
    return direct_ws_bytes(dims);
}

int gato_direct_solve(const gato_dims_t* dims, const float* S, const float* gamma, const float* Qinv,
                      const float* Rinv, const float* Bu, const float* q, const float* r, float* lambda,
                      float* dz, int32_t* flags, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->B == 0) return GATO_OK;  // nothing to do; pointers may be empty
    rc = check_ptrs({S, gamma, Qinv, dyn(Rinv, dims), dyn(Bu, dims), q, dyn(r, dims), lambda, dz, flags});
    if (rc) return rc;
    if (workspace == nullptr || workspace_bytes < direct_ws_bytes(dims)) return GATO_E_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return GATO_E_ALIGN;
    Params p = make_params(dims);
    p.S = const_cast<float*>(S); p.gamma = const_cast<float*>(gamma);
    p.Qinv = const_cast<float*>(Qinv); p.Rinv = const_cast<float*>(Rinv);
    p.Bu = Bu; p.q = q; p.r = r;
    p.lambda = lambda; p.dz = dz; p.flags = flags;
    p.dws = static_cast<float*>(workspace);
    return with_shape(dims->n, dims->m, [&](auto ops) {
        return decltype(ops)::direct(p, stream) == hipSuccess ? GATO_OK : GATO_E_HIP;
    });
}

int32_t gato_cr_levels(int32_t N)
{
    if (N < 1) return 0;
    int levels = 1;
    for (int64_t s = 1; s < N; s *= 2) ++levels;
    return levels;
}

size_t gato_cr_workspace_bytes(const gato_dims_t* dims)
{
    if (check_dims(dims) != GATO_OK || dims->B == 0) return 0;
    return cr_ws_bytes(dims);
}

int gato_cr_solve(const gato_dims_t* dims, const float* S, const float* gamma, const float* Qinv,
                  const float* Rinv, const float* Bu, const float* q, const float* r, float* lambda, float* dz,
                  int32_t* flags, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->B == 0) return GATO_OK;  // nothing to do; pointers may be empty
    rc = check_ptrs({S, gamma, Qinv, dyn(Rinv, dims), dyn(Bu, dims), q, dyn(r, dims), lambda, dz, flags});
    if (rc) return rc;
    if (workspace == nullptr || workspace_bytes < cr_ws_bytes(dims)) return GATO_E_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return GATO_E_ALIGN;
    Params p = make_params(dims);
    p.S = const_cast<float*>(S); p.gamma = const_cast<float*>(gamma);
    p.Qinv = const_cast<float*>(Qinv); p.Rinv = const_cast<float*>(Rinv);
    p.Bu = Bu; p.q = q; p.r = r;
    p.lambda = lambda; p.dz = dz; p.flags = flags;
    p.dws = static_cast<float*>(workspace);
    return cr_launch(p, stream) == hipSuccess ? GATO_OK : GATO_E_HIP;
}

static int check_alpha(const float* alphas_host, int32_t n_alpha, float mu)
{
    if (alphas_host == nullptr) return GATO_E_NULL;
    if (n_alpha < 1 || n_alpha > GATO_MAX_ALPHA) return GATO_E_PARAM;
    if (!(mu >= 0.0f)) return GATO_E_PARAM;
    return GATO_OK;
}

static int merit_call(const gato_dims_t* dims, const float* Q, const float* q, const float* R, const float* r,
                      const float* A, const float* Bu, const float* e, const float* x0, const float* dz,
                      const float* alphas_host, int32_t n_alpha, float mu, float* merit, float* merit0,
                      int32_t* best, int32_t* flags, int32_t variant, int32_t waves, hipStream_t stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if (variant != GATO_MERIT_PER_KNOT && variant != GATO_MERIT_PER_CANDIDATE) return GATO_E_PARAM;
    if (waves < 0 || waves > 16) return GATO_E_PARAM;
    if (dims->B == 0) return GATO_OK;  // nothing to do; pointers may be empty
    rc = check_ptrs({Q, q, dyn(R, dims), dyn(r, dims), dyn(A, dims), dyn(Bu, dims), dyn(e, dims), x0, dz,
                     merit, merit0, best, flags});
    if (rc) return rc;
    rc = check_alpha(alphas_host, n_alpha, mu);
    if (rc) return rc;
    Params p = make_params(dims);
    p.Q = Q; p.q = q; p.R = R; p.r = r; p.A = A; p.Bu = Bu; p.e = e; p.x0 = x0;
    p.dz = const_cast<float*>(dz);
    p.mu = mu; p.n_alpha = n_alpha;
    for (int j = 0; j < n_alpha; ++j) p.alphas[j] = alphas_host[j];
    p.merit = merit; p.merit0 = merit0; p.best = best; p.flags = flags;
    return with_shape(dims->n, dims->m, [&](auto ops) {
        return decltype(ops)::merit(p, stream, variant, waves) == hipSuccess ? GATO_OK : GATO_E_HIP;
    });
}

int gato_merit_eval(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                    const float* r, const float* A, const float* Bu, const float* e,
                    const float* x0, const float* dz, const float* alphas_host, int32_t n_alpha,
                    float mu, float* merit, float* merit0, int32_t* best, int32_t* flags,
                    hipStream_t stream)
{
    return merit_call(dims, Q, q, R, r, A, Bu, e, x0, dz, alphas_host, n_alpha, mu, merit, merit0, best, flags,
                      GATO_MERIT_PER_KNOT, 0, stream);
}

int gato_merit_eval_shape(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                          const float* r, const float* A, const float* Bu, const float* e,
                          const float* x0, const float* dz, const float* alphas_host, int32_t n_alpha,
                          float mu, float* merit, float* merit0, int32_t* best, int32_t* flags,
                          int32_t variant, int32_t waves, hipStream_t stream)
{
    return merit_call(dims, Q, q, R, r, A, Bu, e, x0, dz, alphas_host, n_alpha, mu, merit, merit0, best, flags,
                      variant, waves, stream);
}

int gato_sqp_step_opts(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                       const float* r, const float* A, const float* Bu, const float* e,
                       const float* x0, const float* rho, float eps, int32_t max_iters,
                       const float* alphas_host, int32_t n_alpha, float mu, float* lambda, float* dz,
                       float* merit, float* merit0, int32_t* best, int32_t* iters, float* relres,
                       int32_t* flags, void* workspace, size_t workspace_bytes,
                       gato_stage_times_t* times, const gato_step_opts_t* opts, hipStream_t stream)
{
    int rc = check_dims_step(dims);
    if (rc) return rc;
    if (!native_shape(dims->n, dims->m)) {
        // a shape without kernels of its own: solve the padded problem (padded_dims)
        if (opts && ((opts->solver != GATO_SOLVER_AUTO && opts->solver != GATO_SOLVER_THOMAS &&
                      opts->solver != GATO_SOLVER_CR && opts->solver != GATO_SOLVER_CR_STREAM) ||
                     (opts->refine != 0 && opts->refine != 1)))
            return GATO_E_PARAM;
        if (dims->B == 0) return GATO_OK;
        rc = check_ptrs({Q, q, dyn(R, dims), dyn(r, dims), dyn(A, dims), dyn(Bu, dims), dyn(e, dims), x0, lambda,
                         dz, merit, merit0, best, iters, relres, flags});
        if (rc) return rc;
        if (rho && !aligned4(rho)) return GATO_E_ALIGN;
        if (!(eps > 0.0f) || max_iters < 1) return GATO_E_PARAM;
        rc = check_alpha(alphas_host, n_alpha, mu);
        if (rc) return rc;
        gato_dims_t pd;
        padded_dims(dims, &pd);
        const PadLayout pl = pad_layout(&pd, opts && opts->solver != GATO_SOLVER_AUTO);
        if (workspace == nullptr || workspace_bytes < pl.total) return GATO_E_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return GATO_E_ALIGN;
        char* ws = static_cast<char*>(workspace);
        auto at = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
        const int n = dims->n, m = dims->m, np = pd.n, mp = pd.m, N = dims->N;
        const size_t B = dims->B, Nd = N > 1 ? N - 1 : 0;
        hipError_t e2 = pad_launch(stream, at(pl.Q), Q, B * N, n, n, np, np, 1.0f);
        if (e2 == hipSuccess) e2 = pad_launch(stream, at(pl.q), q, B * N, n, 1, np, 1, 0.0f);
        if (e2 == hipSuccess && Nd) e2 = pad_launch(stream, at(pl.R), R, B * Nd, m, m, mp, mp, 1.0f);
        if (e2 == hipSuccess && Nd) e2 = pad_launch(stream, at(pl.r), r, B * Nd, m, 1, mp, 1, 0.0f);
        if (e2 == hipSuccess && Nd) e2 = pad_launch(stream, at(pl.A), A, B * Nd, n, n, np, np, 0.0f);
        if (e2 == hipSuccess && Nd) e2 = pad_launch(stream, at(pl.Bu), Bu, B * Nd, n, m, np, mp, 0.0f);
        if (e2 == hipSuccess && Nd) e2 = pad_launch(stream, at(pl.e), e, B * Nd, n, 1, np, 1, 0.0f);
        if (e2 == hipSuccess) e2 = pad_launch(stream, at(pl.x0), x0, B, n, 1, np, 1, 0.0f);
        if (e2 == hipSuccess) e2 = pad_launch(stream, at(pl.lam), lambda, B * N, n, 1, np, 1, 0.0f);
        if (e2 != hipSuccess) return GATO_E_HIP;
        rc = gato_sqp_step_opts(&pd, at(pl.Q), at(pl.q), Nd ? at(pl.R) : nullptr, Nd ? at(pl.r) : nullptr,
                                Nd ? at(pl.A) : nullptr, Nd ? at(pl.Bu) : nullptr, Nd ? at(pl.e) : nullptr,
                                at(pl.x0), rho, eps, max_iters, alphas_host, n_alpha, mu, at(pl.lam), at(pl.dz), merit,
                                merit0, best, iters, relres, flags, ws + pl.inner, workspace_bytes - pl.inner, times,
                                opts, stream);
        if (rc != GATO_OK) return rc;
        if (unpad_launch(stream, lambda, at(pl.lam), B * N, n, 1, np, 1) != hipSuccess) return GATO_E_HIP;
        const size_t total = B * ((size_t)N * n + Nd * m);
        const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 4096);
        hipLaunchKernelGGL(k_unpad_dz, dim3(grid), dim3(256), 0, stream, dz, at(pl.dz), (int)B, N, n, m, np, mp);
        return hipGetLastError() == hipSuccess ? GATO_OK : GATO_E_HIP;
    }
    const int solver = opts ? opts->solver : GATO_SOLVER_AUTO;
    const int refine = opts ? opts->refine : 1;
    if (solver != GATO_SOLVER_AUTO && solver != GATO_SOLVER_THOMAS && solver != GATO_SOLVER_CR &&
        solver != GATO_SOLVER_CR_STREAM)
        return GATO_E_PARAM;
    if (refine != 0 && refine != 1) return GATO_E_PARAM;
    if (dims->B == 0) return GATO_OK;  // nothing to do; pointers may be empty
    rc = check_ptrs({Q, q, dyn(R, dims), dyn(r, dims), dyn(A, dims), dyn(Bu, dims), dyn(e, dims), x0, lambda,
                     dz, merit, merit0, best, iters, relres, flags});
    if (rc) return rc;
    if (rho && !aligned4(rho)) return GATO_E_ALIGN;
    if (!(eps > 0.0f) || max_iters < 1) return GATO_E_PARAM;
    rc = check_alpha(alphas_host, n_alpha, mu);
    if (rc) return rc;
    // an explicit solver runs its direct solve at any horizon, the fused ones included
    const bool fused = fused_path(dims) && solver == GATO_SOLVER_AUTO;
    const WsLayout wl = ws_layout(dims);
    if (!fused && dims->B > 0) {
        if (workspace == nullptr || workspace_bytes < wl.total) return GATO_E_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return GATO_E_ALIGN;
    }
    Params p = make_params(dims);
    p.Q = Q; p.q = q; p.R = R; p.r = r; p.A = A; p.Bu = Bu; p.e = e; p.x0 = x0; p.rho = rho;
    p.eps = eps; p.max_iters = max_iters; p.mu = mu; p.n_alpha = n_alpha;
    for (int j = 0; j < n_alpha; ++j) p.alphas[j] = alphas_host[j];
    p.lambda = lambda; p.dz = dz; p.merit = merit; p.merit0 = merit0; p.best = best;
    p.iters = iters; p.relres = relres; p.flags = flags;
    if (!fused) {
        char* ws = static_cast<char*>(workspace);
        p.S = reinterpret_cast<float*>(ws + wl.S);
        p.mpart = reinterpret_cast<float*>(ws + wl.mpart);
        p.gamma = reinterpret_cast<float*>(ws + wl.gamma);
        p.Qinv = reinterpret_cast<float*>(ws + wl.Qinv);
        p.Rinv = reinterpret_cast<float*>(ws + wl.Rinv);
        p.dws = reinterpret_cast<float*>(ws + wl.direct);
    }
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    bool ev_ok = true;
    if (times) {
        for (auto& x : ev) ev_ok = ev_ok && hipEventCreate(&x) == hipSuccess;
        ev_ok = ev_ok && hipEventRecord(ev[0], stream) == hipSuccess;
        if (!ev_ok) {
            for (auto& x : ev)
                if (x) (void)hipEventDestroy(x);
            return GATO_E_HIP;
        }
    }
    rc = with_shape(dims->n, dims->m, [&](auto ops) {
        using O = decltype(ops);
        if (fused) return O::fused(p, stream) == hipSuccess ? GATO_OK : GATO_E_HIP;
        // horizons a workgroup cannot hold: no Phi^-1, since a direct solve follows, and
        // no lower blocks of S when that solve reads only the upper ones
        const bool cr = solver == GATO_SOLVER_AUTO ? cr_preferred(dims, refine != 0) : solver != GATO_SOLVER_THOMAS;
        p.cr_stream = solver == GATO_SOLVER_CR_STREAM;
        p.s_upper_only = cr && !cr_reads_lower(dims, p.cr_stream != 0);
        if (O::form(p, stream, false) != hipSuccess) return GATO_E_HIP;
        if (times && hipEventRecord(ev[1], stream) != hipSuccess) return GATO_E_HIP;
        if (refine && cr && cr_refines_inside(dims, p.cr_stream != 0)) {
            // the solve and its refinement pass in one kernel, on the solve's factors
            if (cr_launch_refined(p, stream) != hipSuccess) return GATO_E_HIP;
        } else if ((cr ? cr_launch(p, stream) : O::direct(p, stream)) != hipSuccess) {
            return GATO_E_HIP;
        } else if (refine) {
            // the correction system: its right-hand side and gamma (S, Q~^-1 and R^-1
            // are the first pass's), its solve, then the sum with the first pass
            char* ws = static_cast<char*>(workspace);
            float* qc = reinterpret_cast<float*>(ws + wl.qc);
            float* rc2 = reinterpret_cast<float*>(ws + wl.rc);
            float* ec = reinterpret_cast<float*>(ws + wl.ec);
            float* x0c = reinterpret_cast<float*>(ws + wl.x0c);
            float* hq = reinterpret_cast<float*>(ws + wl.hq);
            float* tq = reinterpret_cast<float*>(ws + wl.tq);
            Params c = p;
            c.q = qc; c.r = rc2; c.e = ec; c.x0 = x0c;
            c.lambda = reinterpret_cast<float*>(ws + wl.lamc);
            c.dz = reinterpret_cast<float*>(ws + wl.dzc);
            c.flags = reinterpret_cast<int32_t*>(ws + wl.flc);
            const size_t B = dims->B, nlam = B * dims->N * dims->n;
            if (O::residual(p, qc, rc2, ec, x0c, hq, tq, stream) != hipSuccess) return GATO_E_HIP;
            hipLaunchKernelGGL(k_refine_gamma, dim3((unsigned)((nlam + 255) / 256)), dim3(256), 0, stream, c.gamma, hq,
                               tq, ec, x0c, dims->n, dims->N, nlam);
            hipLaunchKernelGGL(k_zero_i32, dim3((dims->B + 255) / 256), dim3(256), 0, stream, c.flags, dims->B);
            if (hipGetLastError() != hipSuccess) return GATO_E_HIP;
            if ((cr ? cr_launch(c, stream) : O::direct(c, stream)) != hipSuccess) return GATO_E_HIP;
            const size_t ndz = B * ((size_t)dims->N * dims->n + (size_t)(dims->N - 1) * dims->m);
            hipLaunchKernelGGL(k_refine_add, dim3(1024), dim3(256), 0, stream, p.lambda, c.lambda, nlam, p.dz, c.dz,
                               ndz, p.flags, c.flags, dims->B);
            if (hipGetLastError() != hipSuccess) return GATO_E_HIP;
        }
        if (times && hipEventRecord(ev[2], stream) != hipSuccess) return GATO_E_HIP;
        if (O::merit_ws(p, stream) != hipSuccess) return GATO_E_HIP;
        return GATO_OK;
    });
    if (times) {
        float t = 0.0f;
        bool ok = rc == GATO_OK && hipEventRecord(ev[3], stream) == hipSuccess &&
                  hipEventSynchronize(ev[3]) == hipSuccess && hipEventElapsedTime(&t, ev[0], ev[3]) == hipSuccess;
        times->total_us = ok ? 1000.0f * t : -1.0f;
        // one fused kernel: the stages are not separable in time
        times->schur_us = times->linsys_us = times->merit_us = -1.0f;
        if (ok && !fused) {
            if (hipEventElapsedTime(&t, ev[0], ev[1]) == hipSuccess) times->schur_us = 1000.0f * t;
            if (hipEventElapsedTime(&t, ev[1], ev[2]) == hipSuccess) times->linsys_us = 1000.0f * t;
            if (hipEventElapsedTime(&t, ev[2], ev[3]) == hipSuccess) times->merit_us = 1000.0f * t;
        }
        for (auto& x : ev) (void)hipEventDestroy(x);
        if (rc == GATO_OK && !ok) rc = GATO_E_HIP;
    }
    return rc;
}

int gato_sqp_step_noalloc(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                          const float* r, const float* A, const float* Bu, const float* e,
                          const float* x0, const float* rho, float eps, int32_t max_iters,
                          const float* alphas_host, int32_t n_alpha, float mu, float* lambda, float* dz,
                          float* merit, float* merit0, int32_t* best, int32_t* iters, float* relres,
                          int32_t* flags, hipStream_t stream)
{
    int rc = check_dims_step(dims);
    if (rc) return rc;
    if (dims->B == 0) return GATO_OK;  // nothing to do; pointers may be empty
    const size_t need = gato_workspace_bytes(dims, n_alpha);
    if (need > (size_t)GATO_NOALLOC_SCRATCH_BYTES) return GATO_E_WORKSPACE;
    void* ws = nullptr;
    size_t wsb = 0;
    if (need > 0) {
        ws = scratch_ptr();
        if (ws == nullptr) return GATO_E_HIP;
        wsb = (size_t)GATO_NOALLOC_SCRATCH_BYTES;
    }
    return gato_sqp_step_opts(dims, Q, q, R, r, A, Bu, e, x0, rho, eps, max_iters, alphas_host, n_alpha, mu, lambda,
                              dz, merit, merit0, best, iters, relres, flags, ws, wsb, nullptr, nullptr, stream);
}

int gato_sqp_step(const gato_dims_t* dims, const float* Q, const float* q, const float* R,
                  const float* r, const float* A, const float* Bu, const float* e,
                  const float* x0, const float* rho, float eps, int32_t max_iters,
                  const float* alphas_host, int32_t n_alpha, float mu, float* lambda, float* dz,
                  float* merit, float* merit0, int32_t* best, int32_t* iters, float* relres,
                  int32_t* flags, void* workspace, size_t workspace_bytes,
                  gato_stage_times_t* times, hipStream_t stream)
{
    return gato_sqp_step_opts(dims, Q, q, R, r, A, Bu, e, x0, rho, eps, max_iters, alphas_host, n_alpha, mu, lambda,
                              dz, merit, merit0, best, iters, relres, flags, workspace, workspace_bytes, times,
                              nullptr, stream);
}

}  // extern "C"
