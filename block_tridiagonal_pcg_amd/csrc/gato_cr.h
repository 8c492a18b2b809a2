// gato_cr.h -- block cyclic reduction of S lambda = gamma as workgroup-level
// device functions: the cyclic-frames elimination plan of the Branch page
// ("Specializing Robotics Solvers in Warp"), the log-depth alternative to the
// block Thomas solve for long horizons.  Same lane layout as gato_stages.h
// (lane i of a knot group holds row i of that knot's blocks).
#pragma once

#include "gato_stages.h"

namespace gato {

// ------------------------------------------------------------------ stage 2, cyclic reduction

// Float4-wide row transfers for the cyclic-reduction workspace (K a multiple
// of 4, rows 16-byte aligned); a masked read takes the zero page instead.
template <int K>
__device__ __forceinline__ void ld4(const float* base, size_t off, bool ok, float* out)
{
    static_assert(K % 4 == 0 && K <= 2048, "");
    const float4* a = reinterpret_cast<const float4*>(ok ? base + off : g_zero_page);
#pragma unroll
    for (int t = 0; t < K / 4; ++t) {
        const float4 f = a[t];
        out[4 * t] = ok ? f.x : 0.0f;
        out[4 * t + 1] = ok ? f.y : 0.0f;
        out[4 * t + 2] = ok ? f.z : 0.0f;
        out[4 * t + 3] = ok ? f.w : 0.0f;
    }
}

template <int K>
__device__ __forceinline__ void st4(float* base, size_t off, const float* v)
{
    static_assert(K % 4 == 0, "");
    float4* a = reinterpret_cast<float4*>(base + off);
#pragma unroll
    for (int t = 0; t < K / 4; ++t) a[t] = make_float4(v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]);
}

// Value of lane P of the knot group, in every lane of the group.
template <int NP, int P>
__device__ __forceinline__ float bcast(float x)
{
    float src = x;
    if constexpr (NP == 32) {
        float lo, hi;
        dup_rows(x, lo, hi);
        src = P < 16 ? lo : hi;
    }
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(src), 0x150 + (P & 15), 0xF, 0xF, false));
}

// acc[c] += acc[c](lane L) * mul for c < K, in place, in chunks of 16 columns.
template <int K, int L>
__device__ __forceinline__ void bcBs_chunks(float* acc, float mul)
{
    if constexpr (K <= 16) {
        BcBs<K>::template run<L>(acc, mul);
    } else {
        BcBs<16>::template run<L>(acc, mul);
        bcBs_chunks<K - 16, L>(acc + 16, mul);
    }
}

// In-place Cholesky factorisation and lower solve of one row-per-lane block
// row [D | R] (D: NC x NC symmetric positive definite in columns 0..NC-1,
// right-hand sides R in columns NC..K-1): afterwards lane i holds row i of
// [C' | C^-1 R] with D = C C' (C lower triangular); only the entries of C' on
// and right of the diagonal are meaningful.  Step j eliminates column j from
// the rows below j (one broadcast multiply-add per remaining column, all lanes
// running one instruction stream) and leaves row j as it is; each row is
// scaled by 1/sqrt(its pivot) once at the end.  (Folding that scaling into the
// step's multiply-add, with multiplier 1/sqrt(pivot) - 1, would cost the row a
// relative error of about 2^-24 sqrt(pivot), which large pivots make visible.)
// `bad` is set when a pivot is not positive or not finite; the factorisation
// then continues, flagged.
template <int NP, int NC, int K, int J = 0>
__device__ __forceinline__ void chol_steps(float* a, int lane, bool active, float& rs_own, bool& bad)
{
    if constexpr (J < NC) {
        const float piv = bcast<NP, J>(a[J]);
        bad |= active && (!(piv > 0.0f) || !__builtin_isfinite(piv));
        const float rinv = __builtin_amdgcn_rcpf(piv);  // v_rcp_f32, 1 ulp
        const float g = (active && lane > J) ? -(a[J] * rinv) : 0.0f;
        rs_own = (active && lane == J) ? __builtin_amdgcn_rsqf(piv) : rs_own;  // v_rsq_f32, 1 ulp
        if constexpr (NP == 16) {
            bcBs_chunks<K - J, J>(a + J, g);
        } else {
            BcRow<32, K - J> src(a + J);
            axpyb<32, K - J, J>(a + J, src, g);
        }
        chol_steps<NP, NC, K, J + 1>(a, lane, active, rs_own, bad);
    }
}

// Groups with `active` false run the same instructions with zero multipliers
// and a unit scale, which leaves their rows exactly as they were (their own
// rows are the only broadcast sources they read).
template <int NP, int NC, int K>
__device__ __forceinline__ void chol_solve(float* a, int lane, bool& bad, bool active = true)
{
    float rs = 1.0f;
    chol_steps<NP, NC, K>(a, lane, active, rs, bad);
#pragma unroll
    for (int c = 0; c < K; ++c) a[c] *= rs;
}

// Back substitution C' x = v for the factor left by chol_solve: lane i holds
// row i of C' (ct) and v_i; on return x holds x_i.  Runs from the last row up,
// one broadcast per row.
template <int NP, int NC, int P = NC - 1>
__device__ __forceinline__ void tri_upper_solve(const float* ct, float v, float dinv, int lane, float& x)
{
    if constexpr (P >= 0) {
        const float xp = bcast<NP, P>(v * dinv);
        if (lane == P) x = xp;
        v = lane < P ? fmaf(-ct[P], xp, v) : v;
        tri_upper_solve<NP, NC, P - 1>(ct, v, dinv, lane, x);
    }
}

// Forward substitution C x = v with the same factor, lane i holding row i of C
// (column i of C': cl[c] = C'[c][i], zero for c > i) and v_i; on return x
// holds x_i.  Runs from the first row down, one broadcast per row.
template <int NP, int NC, int P = 0>
__device__ __forceinline__ void tri_lower_solve(const float* cl, float v, float dinv, int lane, float& x)
{
    if constexpr (P < NC) {
        const float xp = bcast<NP, P>(v * dinv);
        if (lane == P) x = xp;
        v = lane > P ? fmaf(-cl[P], xp, v) : v;
        tri_lower_solve<NP, NC, P + 1>(cl, v, dinv, lane, x);
    }
}

// What lane i reads for the recovery of knot k's dz besides its row of
// S_{k,k+1}: its rows of Q~^-1 and R^-1, column i of B_k, q_i and r_i.  ok
// false reads zeros (k must still be a knot of the horizon).
template <class SH>
struct RecRows {
    float qi[SH::NC], ri[SH::MC], bc[SH::NC], qv, rv;
};

template <class SH>
__device__ __forceinline__ void rec_load(const Params& p, int b, int k, int i, bool ok, RecRows<SH>& r)
{
    constexpr int NC = SH::NC, MC = SH::MC;
    const Ix<SH> ix{p.N};
    const bool rowv = ok && i < NC;
    const bool urow = ok && k < p.N - 1 && i < MC;
    ld_row<NC>(p.Qinv, ix.Q(b, k, i), rowv, r.qi);
    ld_row<MC>(p.Rinv, ix.R(b, k, i), urow, r.ri);
    ld_row<NC, MC>(p.Bu, ix.Bu(b, k, 0) + i, urow, r.bc);  // column i of B_k
    r.qv = ld1(p.q, ix.vn(b, k, i), rowv);
    r.rv = ld1(p.r, ix.vm(b, k, i), urow);
}

// The recovery of knot k's dz (recover(), the back substitution of the Schur
// solve) from lambda_k and lambda_{k+1} in lane i's row, given the rows
// rec_load read and lane i's row of S_{k,k+1} (sup); ok false masks the stores.
template <class SH>
__device__ __forceinline__ void rec_store(const Params& p, int b, int k, int i, bool ok, const RecRows<SH>& r,
                                          const float* sup, float lam, float lamn)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC;
    const Ix<SH> ix{p.N};
    const bool rowv = ok && i < NC;
    const bool urow = ok && k < p.N - 1 && i < MC;
    float h = 0.0f;  // (Q~_k^-1 q_k)_i, as the formation forms it
    dotb<NP, NC>(h, Bc<NP>(r.qv), r.qi);
    float dx, du;
    recover<SH>(i, rowv, urow, rowv ? lam : 0.0f, lamn, r.qi, sup, h, r.bc, r.rv, r.ri, dx, du);
    if (rowv) p.dz[ix.dx(b, k, i)] = dx;
    if (urow) p.dz[ix.du(b, k, i)] = du;
}

// Both together, with the row of S_{k,k+1} read here too; ok false masks the
// loads and the stores.
template <class SH>
__device__ __forceinline__ void recover_knot(const Params& p, int b, int k, int i, bool ok, float lam, float lamn)
{
    constexpr int NC = SH::NC;
    const Ix<SH> ix{p.N};
    RecRows<SH> r;
    rec_load<SH>(p, b, k, i, ok, r);
    float sup[NC];
    ld_row<NC>(p.S, ix.blk(b, k, 2, i), ok && i < NC, sup);
    rec_store<SH>(p, b, k, i, ok, r, sup, lam, lamn);
}

// One knot's row of the reduced system in the workspace, padded to whole
// float4s.  A knot still in the system keeps [- | U | gamma | D]; when it is
// eliminated the row becomes [W1 | W2 | w3 | C'] (see cr_solve).
template <class SH>
struct CrRow {
    static constexpr int NC = SH::NC;
    static constexpr int L = 0, U = NC, G = 2 * NC, D = 2 * NC + 1;
    static constexpr int W = (3 * NC + 1 + 3) / 4 * 4;
};

// Block cyclic reduction of S lambda = gamma, then the recovery of dz: the
// cyclic-frames elimination plan of the Branch page ("Specializing Robotics
// Solvers in Warp": the elimination-plan figure of "The three descriptions" and
// the cyclic-reduction row of the plans table), odd knots first, then every
// other knot of what remains, ceil(log2 N) + 1 levels in all.  Each
// elimination is the factor step that page describes for its cyclic fronts:
// an in-place Cholesky factorisation and lower solve, then a Schur-complement
// update of the neighbours.
//
// Level l works on the knots that are multiples of s = 2^l.  With U_k the
// coupling of knot k to knot k + s in that system (and U_{k-s}' its coupling
// to k - s), every knot j eliminated at this level (an odd multiple of s)
// factors D_j = C_j C_j' and forms
//   W1_j = C_j^-1 U_{j-s}',  W2_j = C_j^-1 U_j,  w3_j = C_j^-1 gamma_j,
// and every kept knot i (a multiple of 2s) takes the Schur complement of its
// two eliminated neighbours:
//   D_i <- D_i - W2_{i-s}' W2_{i-s} - W1_{i+s}' W1_{i+s},   U_i <- -W1_{i+s}' W2_{i+s},
//   gamma_i <- gamma_i - W2_{i-s}' w3_{i-s} - W1_{i+s}' w3_{i+s},
// so the kept knots form a system of the same kind on stride 2s, symmetric by
// construction.  The last level solves knot 0 alone, and the back
// substitution runs the levels in reverse:
//   lambda_j = C_j'^-1 (w3_j - W1_j lambda_{j-s} - W2_j lambda_{j+s}).
// This is the block Cholesky factorisation of S with its knots reordered, so
// every pivot block is SPD when S is; a pivot that is not positive sets
// S_NOT_SPD.
//
// One workgroup holds one solve; its lane groups (lane i: row i of a block)
// share each level's eliminations and then its updates, with a workgroup
// barrier between the two phases.  The products W'W take column i of W (a
// strided read of the eliminated knot's workspace rows) and broadcast rows of
// W, so no transpose is formed.  Level 0 reads S and gamma directly; later
// levels, the factors and the back substitution use the workspace rows.
// Waves with no knot in a phase skip it.
template <class SH>
__device__ __forceinline__ void cr_solve(const Params& p, int b)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC;
    using RW = CrRow<SH>;
    constexpr int W = RW::W;
    constexpr int KA = 3 * NC + 1;  // [D | U_{j-s}' | U_j | gamma]
    const Ix<SH> ix{p.N};
    const int N = p.N;
    const int i = threadIdx.x % NP;
    const int g = threadIdx.x / NP;
    const int G = blockDim.x / NP;
    const bool rowi = i < NC;
    float* ws = p.dws;
    auto wrow = [&](int k, int r) { return (((size_t)b * N + k) * NC + r) * W; };

    __shared__ int wg_flags;
    if (threadIdx.x == 0) wg_flags = 0;
    __syncthreads();  // the flag word is zero before any wave can set a bit in it
    bool bad = false, nonfinite = false;

    int levels = 0;
    for (int s = 1; s < N; s *= 2, ++levels) {
        const bool fromS = s == 1;
        // eliminate the odd multiples of s
        const int E = (N + s - 1) / (2 * s);
        for (int t0 = 0; t0 < E; t0 += G) {
            const int t = t0 + g;
            const bool ok = t < E;
            if (__builtin_amdgcn_ballot_w64(ok) == 0) continue;
            const int j = ok ? s * (2 * t + 1) : s;
            const bool hasU = j + s < N;
            const bool ld = ok && rowi;
            float a[KA];
            float* D = a;
            float* Lt = a + NC;      // row i of U_{j-s}'
            float* U = a + 2 * NC;
            if (fromS) {
                ld_row<NC>(p.S, ix.blk(b, j, 1, i), ld, D);
                ld_row<NC>(p.S, ix.blk(b, j, 0, i), ld, Lt);
                ld_row<NC>(p.S, ix.blk(b, j, 2, i), ld && hasU, U);
                a[3 * NC] = ld1(p.gamma, ix.vn(b, j, i), ld);
            } else {
                float r[W];
                ld4<W>(ws, wrow(j, i), ld, r);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    D[c] = r[RW::D + c];
                    U[c] = hasU ? r[RW::U + c] : 0.0f;
                }
                a[3 * NC] = r[RW::G];
                ld_row<NC, W>(ws, wrow(j - s, 0) + RW::U + i, ld, Lt);  // column i of U_{j-s}
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) D[c] = ok ? D[c] : (c == i ? 1.0f : 0.0f);  // absent: identity
            bool bk = false;
            chol_solve<NP, NC, KA>(a, i, bk);
            bad |= bk && ok;
            if (ld) {
                float r[W];
#pragma unroll
                for (int c = 0; c < W; ++c) r[c] = 0.0f;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    r[RW::L + c] = Lt[c];  // W1
                    r[RW::U + c] = U[c];   // W2
                    r[RW::D + c] = D[c];   // row i of C'
                }
                r[RW::G] = a[3 * NC];  // w3
                st4<W>(ws, wrow(j, i), r);
            }
        }
        __syncthreads();
        // update the multiples of 2s from their eliminated neighbours
        const int K = (N + 2 * s - 1) / (2 * s);
        for (int t0 = 0; t0 < K; t0 += G) {
            const int t = t0 + g;
            const bool ok = t < K;
            if (__builtin_amdgcn_ballot_w64(ok) == 0) continue;
            const int k = ok ? 2 * s * t : 0;
            const bool hasL = k > 0, hasU = k + s < N;
            const bool ld = ok && rowi;
            float D[NC], U[NC], gam;
            if (fromS) {
                ld_row<NC>(p.S, ix.blk(b, k, 1, i), ld, D);
                gam = ld1(p.gamma, ix.vn(b, k, i), ld);
            } else {
                float r[W];
                ld4<W>(ws, wrow(k, i), ld, r);
#pragma unroll
                for (int c = 0; c < NC; ++c) D[c] = r[RW::D + c];
                gam = r[RW::G];
            }
            {
                // knot k - s: D -= W2' W2, gamma -= W2' w3
                const int km = hasL ? k - s : 0;
                float col[NC], row[NC];
                ld_row<NC, W>(ws, wrow(km, 0) + RW::U + i, ld && hasL, col);  // column i of W2
                ld_row<NC>(ws, wrow(km, i) + RW::U, ld && hasL, row);          // row i of W2
                const float w3 = ld1(ws, wrow(km, i) + RW::G, ld && hasL);
#pragma unroll
                for (int c = 0; c < NC; ++c) col[c] = -col[c];
                gemm_rows<NP, NC, NC>(D, BcRow<NP, NC>(row), col);
                dotb<NP, NC>(gam, Bc<NP>(w3), col);
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) U[c] = 0.0f;
            {
                // knot k + s: D -= W1' W1, U = -W1' W2, gamma -= W1' w3
                const int kp = hasU ? k + s : 0;
                float col[NC], r1[NC], r2[NC];
                ld_row<NC, W>(ws, wrow(kp, 0) + RW::L + i, ld && hasU, col);  // column i of W1
                ld_row<NC>(ws, wrow(kp, i) + RW::L, ld && hasU, r1);           // row i of W1
                ld_row<NC>(ws, wrow(kp, i) + RW::U, ld && hasU, r2);           // row i of W2
                const float w3 = ld1(ws, wrow(kp, i) + RW::G, ld && hasU);
#pragma unroll
                for (int c = 0; c < NC; ++c) col[c] = -col[c];
                gemm_rows<NP, NC, NC>(D, BcRow<NP, NC>(r1), col);
                gemm_rows<NP, NC, NC>(U, BcRow<NP, NC>(r2), col);
                dotb<NP, NC>(gam, Bc<NP>(w3), col);
            }
            if (ld) {
                float r[W];
#pragma unroll
                for (int c = 0; c < W; ++c) r[c] = 0.0f;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    r[RW::U + c] = U[c];
                    r[RW::D + c] = D[c];
                }
                r[RW::G] = gam;
                st4<W>(ws, wrow(k, i), r);
            }
        }
        __syncthreads();
    }

    // last level: knot 0 alone, lambda_0 = C_0'^-1 C_0^-1 gamma_0
    {
        const bool ok = g == 0;
        if (__builtin_amdgcn_ballot_w64(ok) != 0) {
            const bool ld = ok && rowi;
            float a[NC + 1];
            if (N == 1) {
                ld_row<NC>(p.S, ix.blk(b, 0, 1, i), ld, a);
                a[NC] = ld1(p.gamma, ix.vn(b, 0, i), ld);
            } else {
                float r[W];
                ld4<W>(ws, wrow(0, i), ld, r);
#pragma unroll
                for (int c = 0; c < NC; ++c) a[c] = r[RW::D + c];
                a[NC] = r[RW::G];
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) a[c] = ok ? a[c] : (c == i ? 1.0f : 0.0f);
            bool bk = false;
            chol_solve<NP, NC, NC + 1>(a, i, bk);
            bad |= bk && ok;
            float dg = 1.0f;  // C_0'[i][i]
#pragma unroll
            for (int c = 0; c < NC; ++c) dg = c == i ? a[c] : dg;
            float lam = 0.0f;
            tri_upper_solve<NP, NC>(a, a[NC], __builtin_amdgcn_rcpf(ld ? dg : 1.0f), i, lam);
            nonfinite |= ld && !__builtin_isfinite(lam);
            if (ld) p.lambda[ix.vn(b, 0, i)] = lam;
        }
        __syncthreads();
    }

    // back substitution, levels in reverse
    for (int l = levels - 1; l >= 0; --l) {
        const int s = 1 << l;
        const int E = (N + s - 1) / (2 * s);
        for (int t0 = 0; t0 < E; t0 += G) {
            const int t = t0 + g;
            const bool ok = t < E;
            if (__builtin_amdgcn_ballot_w64(ok) == 0) continue;
            const int j = ok ? s * (2 * t + 1) : s;
            const bool hasU = j + s < N;
            const bool ld = ok && rowi;
            float r[W];
            ld4<W>(ws, wrow(j, i), ld, r);
            const float lm = ld1(p.lambda, ix.vn(b, j - s, i), ld);
            const float lp = ld1(p.lambda, ix.vn(b, hasU ? j + s : j, i), ld && hasU);
            float v = r[RW::G];
            float acc = 0.0f;
            dotb<NP, NC>(acc, Bc<NP>(lm), r + RW::L);  // W1_j lambda_{j-s}
            dotb<NP, NC>(acc, Bc<NP>(lp), r + RW::U);  // W2_j lambda_{j+s}
            v -= acc;
            float dg = 1.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) dg = c == i ? r[RW::D + c] : dg;
            float lam = 0.0f;
            tri_upper_solve<NP, NC>(r + RW::D, v, __builtin_amdgcn_rcpf(ld ? dg : 1.0f), i, lam);
            nonfinite |= ld && !__builtin_isfinite(lam);
            if (ld) p.lambda[ix.vn(b, j, i)] = lam;
        }
        __syncthreads();
    }

    // recovery of every knot's dz from lambda_k and lambda_{k+1}
    for (int t0 = 0; t0 < N; t0 += G) {
        const int k = t0 + g;
        const bool ok = k < N;
        if (__builtin_amdgcn_ballot_w64(ok) == 0) continue;
        const int kk = ok ? k : 0;
        const bool rowv = ok && rowi;
        const float lam = ld1(p.lambda, ix.vn(b, kk, i), rowv);
        const float lamn = ld1(p.lambda, ix.vn(b, kk + 1 < N ? kk + 1 : kk, i), rowv && kk + 1 < N);
        recover_knot<SH>(p, b, kk, i, ok, lam, lamn);
    }

    // per-solve flags: any lane of the workgroup (an LDS atomic, then one writer)
    const int fl = (bad ? GATO_F_S_NOT_SPD : 0) | (nonfinite ? GATO_F_NONFINITE : 0);
    if (fl) atomicOr(&wg_flags, fl);
    __syncthreads();
    if (threadIdx.x == 0) {
        p.flags[b] |= wg_flags;
        if (p.iters) p.iters[b] = 0;
        if (p.relres) p.relres[b] = 0.0f;
    }
}

// ------------------------------------------------------------------ cyclic reduction, register-resident

// The same elimination for horizons whose knots fit in one workgroup's
// registers (N <= 128, n <= 16): lane group g keeps the odd knot 2g+1 and one
// even knot for the whole solve, so only the W blocks of eliminated knots move
// between groups, through LDS, and memory sees S and the recovery's inputs
// once.  Even knot 2m is eliminated at level 1 + ctz(m) (knot 0 last); the even
// knots are assigned to groups in order of decreasing level, so each level's
// eliminations and updates fall on contiguous groups:
//   group 0: knot 0;  then the knots of the deepest level, ..., then those of
//   level 1, each level in increasing knot order.
// With M even knots, c(t) = (M - 1) >> t of m = 1 .. M-1 are multiples of 2^t,
// and the m with ctz(m) = t occupy groups [1 + c(t+1), 1 + c(t)).
__host__ __device__ constexpr int cr_mult(int M, int t) { return (M - 1) >> t; }

__host__ __device__ constexpr int cr_even_group(int m, int M)
{
    if (m == 0) return 0;
    int t = 0;
    while (((m >> t) & 1) == 0) ++t;
    return 1 + cr_mult(M, t + 1) + ((m >> t) - 1) / 2;
}

// Inverse of cr_even_group for 0 <= g < M.
__host__ __device__ constexpr int cr_group_even(int g, int M)
{
    if (g <= 0) return 0;
    for (int t = 0; t < 31; ++t) {
        const int lo = 1 + cr_mult(M, t + 1), hi = 1 + cr_mult(M, t);
        if (g >= lo && g < hi) return (2 * (g - lo) + 1) << t;
    }
    return 0;
}

// Nested dissection for horizons beyond one workgroup's registers (n <= 16,
// N > 128): the knots are cut into ND_CHUNKS contiguous chunks, one per lane
// group; each chunk's interior knots are eliminated in order (k_nd_reduce),
// which leaves a block-tridiagonal system on the chunks' first and last knots
// (2 * ND_CHUNKS of them); that system is reduced cyclically by the
// register-resident kernel in its "virtual" mode; the interior knots are then
// back-substituted chunk by chunk (k_nd_back).  Workspace, in floats:
//   [B][N][FW]       the factor of each interior knot: rows [W1 | w3] (n x R1),
//                    then C' packed by rows from the diagonal on (TRI)
//   [B][2C][n][W]    rows [L | U | gamma | D] of the boundary system
//   [B][C][n][16]    C' rows of the boundary system's odd knots
// (C = ND_CHUNKS, W = CrRow<SH>::W).  W2 = C^-1 U_f is not kept: the back
// substitution applies C^-1 to U_f lambda_{f+1}, with U_f read from S again,
// which costs one more triangular solve and saves a third of the factor's bytes.
constexpr int ND_CHUNKS = 64;
// The chunk kernels spread one solve's chunks over ND_SPLIT workgroups of
// ND_GPW lane groups each (workgroup y of solve b: chunks y*ND_GPW ..
// (y+1)*ND_GPW - 1), so that batches smaller than the device still fill it:
// four 256-thread workgroups per solve measure like two 512-thread ones at
// B = 128 and are 16-22 % faster at B = 32 and 64.
#ifndef GATO_ND_SPLIT
#define GATO_ND_SPLIT 4
#endif
constexpr int ND_SPLIT = GATO_ND_SPLIT;
constexpr int ND_GPW = ND_CHUNKS / ND_SPLIT;
static_assert(ND_CHUNKS % ND_SPLIT == 0 && ND_GPW % 4 == 0, "whole waves per workgroup");

__host__ __device__ constexpr int nd_start(int j, int N) { return (int)(((long long)j * N) / ND_CHUNKS); }

// Real knot of boundary-system knot v: chunk v/2's first (v even) or last (v odd) knot.
__host__ __device__ constexpr int nd_real(int v, int N)
{
    return (v & 1) ? nd_start(v / 2 + 1, N) - 1 : nd_start(v / 2, N);
}

// Floats of one interior knot's factor: n rows [W1 | w3] of R1 = round4(n + 1),
// then the n (n + 1) / 2 entries of C' on and right of its diagonal, row after
// row (row i from offset nd_tri_off(i, n)), padded to a float4.
__host__ __device__ constexpr int nd_r1(int n) { return (n + 1 + 3) / 4 * 4; }
__host__ __device__ constexpr int nd_tri_off(int i, int n) { return i * n - i * (i - 1) / 2; }
__host__ __device__ constexpr int nd_fac_floats(int n) { return n * nd_r1(n) + (n * (n + 1) / 2 + 3) / 4 * 4; }

template <class SH>
struct NdWs {
    static constexpr int NC = SH::NC, W = CrRow<SH>::W, R1 = nd_r1(NC), FW = nd_fac_floats(NC);
    size_t B, N;
    __host__ __device__ size_t fac(size_t b, size_t k, size_t i) const { return (b * N + k) * FW + i * R1; }
    __host__ __device__ size_t tri(size_t b, size_t k) const { return (b * N + k) * FW + NC * R1; }
    __host__ __device__ size_t vrow(size_t b, size_t v, size_t i) const
    {
        return B * N * FW + ((b * 2 * ND_CHUNKS + v) * NC + i) * W;
    }
    __host__ __device__ size_t oc(size_t b, size_t g, size_t i) const
    {
        return B * (N * FW + 2 * ND_CHUNKS * NC * W) + ((b * ND_CHUNKS + g) * NC + i) * 16;
    }
    __host__ __device__ size_t floats() const { return B * (N * FW + 2 * ND_CHUNKS * NC * W) + B * ND_CHUNKS * NC * 16; }
};

template <class SH>
struct CrResLds {
    static constexpr int NC = SH::NC, YW = 2 * NC + 1;
    static constexpr int MAXG = 64;
    float os[MAXG][NC][YW];  // [W1 | W2 | w3] rows of the odd knots (level 0), kept to the end
    union {
        float es[MAXG / 2][NC][YW];  // [W1 | W2 | w3] rows of the even knots eliminated at one level
        struct {
            float lam[2 * MAXG][NC];  // lambda, once the forward sweep is over
            // the in-kernel refinement pass: the first pass's dx_k and du_k, and
            // t_k and e'_k less its dx_{k+1} term, which knot k + 1's gamma' takes
            float dx[2 * MAXG][NC];
            float du[2 * MAXG][SH::MC];
            float ex[2 * MAXG][NC];
            double epd[2 * MAXG][NC];
        };
    };
    int flags;
};

// VIRT: solve the boundary system of the nested dissection (2 * ND_CHUNKS knots,
// rows from the workspace) and write its lambda at the real knots, instead of
// solving S itself and recovering dz.
// REF: follow the solve with one pass of iterative refinement of the KKT
// system (kkt_rows) inside the kernel: the first pass's lambda and dz stay in
// registers, the residual in double gives the correction's gamma' (formed as
// the formation forms gamma), and the correction is solved with the factors the
// first pass left (C' and the W rows of every eliminated knot: the odd knots'
// in LDS and the workspace, the even knots' in registers), by a second sweep
// over the same levels on the right-hand side alone (w3' = C^-1 gamma' by
// forward substitution, the kept knots' gamma' less W2' w3' and W1' w3') and a
// second back substitution.  lambda and dz are the sums of the two passes.
template <class SH, bool VIRT = false, bool REF = false>
__device__ __forceinline__ void cr_resident(const Params& p, int b)
{
    static_assert(!(VIRT && REF), "the refinement pass is for the whole solve");
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC;
    static_assert(NP == 16, "one knot row per lane of a 16-lane group");
    using LDS = CrResLds<SH>;
    constexpr int YW = LDS::YW;
    constexpr int KA = 3 * NC + 1;  // [D | L | U | gamma]
    constexpr int W = CrRow<SH>::W;
    using RW = CrRow<SH>;
    __shared__ LDS sm;
    const Ix<SH> ix{p.N};
    const NdWs<SH> nw{(size_t)p.B, (size_t)p.N};
    const int N = VIRT ? 2 * ND_CHUNKS : p.N;
    const int M = (N + 1) / 2;  // even knots, one per lane group
    // lane indices (formed again from the thread index after the forward sweep)
    int i = threadIdx.x % NP;
    int g = threadIdx.x / NP;
    bool rowi = i < NC;
    int ii = rowi ? i : 0;  // LDS row index that stays inside a slot
    bool hasG = g < M;
    int levels = 0;  // reduction levels, ceil(log2 N)
    for (int s = 1; s < N; s *= 2) ++levels;
    int jo = 2 * g + 1;  // this group's odd knot
    bool hasO = hasG && jo < N;
    int me = hasG ? cr_group_even(g, M) : 0;
    int ke = 2 * me;  // this group's even knot
    int lev = me == 0 ? levels : 1 + __builtin_ctz(me);  // its elimination level (levels: the last solve)

    if (threadIdx.x == 0) sm.flags = 0;
    __syncthreads();  // the flag word is zero before any wave can set a bit in it
    bool bad = false, nonfinite = false;
    // stage-ordered wave priorities (wave_prio) in level 0 and the recoveries
    wave_prio<true, 3>();

    // level 0, eliminations: the odd knots; their W rows go to LDS, and their C'
    // rows, needed only by the last back-substitution step, to the workspace
    // (16 floats per row, M knots per solve)
    const size_t ocrow = VIRT ? nw.oc(b, hasO ? g : 0, ii) : (((size_t)b * M + (hasO ? g : 0)) * NC + ii) * 16;
    // REF: the even knots' C' rows go to the workspace too, after the odd knots'
    // (row i of group g's even knot at ec_at(b, g) + 16 i), and q' and r' after them
    const size_t ec0 = (size_t)p.B * M * NC * 16;
    auto ec_at = [&](int bb, int gg) { return ec0 + ((size_t)bb * M + gg) * NC * 16; };
    {
        const bool ld = hasO && rowi;
        const int jj = hasO ? jo : 0;
        float a[KA];
        if constexpr (VIRT) {
            float r[W];
            ld4<W>(p.dws, nw.vrow(b, jj, ii), ld, r);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                a[c] = r[RW::D + c];
                a[NC + c] = r[RW::L + c];
                a[2 * NC + c] = jo + 1 < N ? r[RW::U + c] : 0.0f;
            }
            a[3 * NC] = r[RW::G];
        } else {
            ld_row<NC>(p.S, ix.blk(b, jj, 1, i), ld, a);
            // L = S_{j,j-1} = S_{j-1,j}': column i of the upper block of knot j - 1
            ld_row<NC, NC>(p.S, ix.blk(b, jj > 0 ? jj - 1 : 0, 2, 0) + ii, ld, a + NC);
            ld_row<NC>(p.S, ix.blk(b, jj, 2, i), ld && jo + 1 < N, a + 2 * NC);
            a[3 * NC] = ld1(p.gamma, ix.vn(b, jj, i), ld);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) a[c] = hasO ? a[c] : (c == i ? 1.0f : 0.0f);
        if (__builtin_amdgcn_ballot_w64(hasO) != 0) {
            chol_solve<NP, NC, KA>(a, i, bad, hasO);
            wave_prio<true, 1>();
            if (ld) {
#pragma unroll
                for (int c = 0; c < YW; ++c) sm.os[g][i][c] = a[NC + c];
                float r[16];
#pragma unroll
                for (int c = 0; c < 16; ++c) r[c] = c < NC ? a[c] : 0.0f;
                st4<16>(p.dws, ocrow, r);
            }
        }
    }

    // even knot: [D | L | U | gamma] until it is eliminated, then [C' | W1 | W2 | w3]
    float e[KA];
    {
        const bool ld = hasG && rowi;
        if constexpr (VIRT) {
            float r[W];
            ld4<W>(p.dws, nw.vrow(b, ke, ii), ld, r);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                e[c] = r[RW::D + c];
                e[2 * NC + c] = ke + 1 < N ? r[RW::U + c] : 0.0f;
            }
            e[3 * NC] = r[RW::G];
        } else {
            ld_row<NC>(p.S, ix.blk(b, ke, 1, i), ld, e);
            ld_row<NC>(p.S, ix.blk(b, ke, 2, i), ld && ke + 1 < N, e + 2 * NC);
            e[3 * NC] = ld1(p.gamma, ix.vn(b, ke, i), ld);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) e[NC + c] = 0.0f;
    }
    wave_prio<true, 0>();
    __syncthreads();

    // Schur update of a kept knot from the W rows of its eliminated neighbours
    // (Wm: knot k - s, Wp: knot k + s; either absent at the ends), and, when the
    // knot is eliminated at the next level, its coupling to knot k - 2s there.
    auto update = [&](bool kept, bool hasL, bool hasU, bool needL, const float* Wm, const float* Wp) {
        // every value read from an absent neighbour's slot is masked to zero
        // (a slot that no knot wrote may hold any bits)
        const bool okm = kept && hasL, okp = kept && hasU;
        if constexpr (SH::MMA && NC < 16) {
            // On the matrix cores every product is (columns)' (columns): lane c
            // reads column c of the W blocks from LDS, and lane n reads w3, so
            // the sum's column n is the gamma update.  Rows of a group that
            // sits out come out as zero, and padding lanes keep their rows.
            const int c2 = i <= NC ? NC + i : 0;   // W2 columns, w3 at lane n
            const int c1 = i < NC ? i : 2 * NC;    // W1 columns, w3 at lane n
            const bool cl = i <= NC;
            float m2[NC], p1[NC], r[NC + 1];
#pragma unroll
            for (int l = 0; l < NC; ++l) {
                m2[l] = (okm && cl) ? Wm[l * YW + c2] : 0.0f;
                p1[l] = (okp && cl) ? Wp[l * YW + c1] : 0.0f;
            }
            // D -= W2m' W2m + W1p' W1p, gamma -= W2m' w3m + W1p' w3p
            mma16_t acc = {};
            mma_abt<NC>(acc, m2, m2);
            mma_abt<NC>(acc, p1, p1);
            mma_rows<NC + 1>(acc, r);
#pragma unroll
            for (int c = 0; c < NC; ++c) e[c] = rowi ? e[c] - r[c] : e[c];
            e[3 * NC] = rowi ? e[3 * NC] - r[NC] : e[3 * NC];
            // U = -W1p' W2p (the old U is not needed: W1p already carries it)
            {
                float p2[NC];
#pragma unroll
                for (int l = 0; l < NC; ++l) p2[l] = (okp && rowi) ? Wp[l * YW + NC + ii] : 0.0f;
                mma16_t au = {};
                mma_abt<NC>(au, p1, p2);
                mma_rows<NC>(au, r);
#pragma unroll
                for (int c = 0; c < NC; ++c) e[2 * NC + c] = kept ? (rowi ? 0.0f - r[c] : 0.0f) : e[2 * NC + c];
            }
            // L = -W2m' W1m when the knot is eliminated next (the old L is not needed)
            if (__builtin_amdgcn_ballot_w64(needL) != 0) {
                float m1[NC];
#pragma unroll
                for (int l = 0; l < NC; ++l) m1[l] = (okm && rowi) ? Wm[l * YW + ii] : 0.0f;
                mma16_t al = {};
                mma_abt<NC>(al, m2, m1);
                mma_rows<NC>(al, r);
#pragma unroll
                for (int c = 0; c < NC; ++c) e[NC + c] = kept ? (rowi ? 0.0f - r[c] : 0.0f) : e[NC + c];
            }
            return;
        }
        float col[NC], row[NC];
        // D -= W2m' W2m, gamma -= W2m' w3m, and L = -W2m' W1m when needed
#pragma unroll
        for (int m = 0; m < NC; ++m) col[m] = (okm && rowi) ? -Wm[m * YW + NC + ii] : 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) row[c] = okm ? Wm[ii * YW + NC + c] : 0.0f;
        gemm_rows<NP, NC, NC>(e, BcRow<NP, NC>(row), col);
        dotb<NP, NC>(e[3 * NC], Bc<NP>(okm ? Wm[ii * YW + 2 * NC] : 0.0f), col);
        if (__builtin_amdgcn_ballot_w64(needL) != 0) {
            // the old L is not needed: a kept knot's L only matters at its elimination
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                row[c] = okm ? Wm[ii * YW + c] : 0.0f;
                e[NC + c] = kept ? 0.0f : e[NC + c];
            }
            gemm_rows<NP, NC, NC>(e + NC, BcRow<NP, NC>(row), col);
        }
        // D -= W1p' W1p, U = -W1p' W2p, gamma -= W1p' w3p
#pragma unroll
        for (int m = 0; m < NC; ++m) col[m] = (okp && rowi) ? -Wp[m * YW + ii] : 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) row[c] = okp ? Wp[ii * YW + c] : 0.0f;
        gemm_rows<NP, NC, NC>(e, BcRow<NP, NC>(row), col);
        // the old U is not needed either (W1p already carries it)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            row[c] = okp ? Wp[ii * YW + NC + c] : 0.0f;
            e[2 * NC + c] = kept ? 0.0f : e[2 * NC + c];
        }
        gemm_rows<NP, NC, NC>(e + 2 * NC, BcRow<NP, NC>(row), col);
        dotb<NP, NC>(e[3 * NC], Bc<NP>(okp ? Wp[ii * YW + 2 * NC] : 0.0f), col);
    };

    // level 0, updates: every even knot, from odd knots k - 1 (group m - 1) and k + 1 (group m)
    {
        const bool kept = hasG;
        if (__builtin_amdgcn_ballot_w64(kept) != 0) {
            const bool hasL = ke > 0, hasU = ke + 1 < N;
            const float* Wm = &sm.os[hasL ? me - 1 : 0][0][0];
            const float* Wp = &sm.os[hasU ? me : 0][0][0];
            update(kept, hasL, hasU, kept && lev == 1, Wm, Wp);
        }
    }
    __syncthreads();

    // levels 1 .. levels-1: the even knots of that level are eliminated, the rest updated
    for (int l = 1; l < levels; ++l) {
        const int s = 1 << l;
        const int first = 1 + cr_mult(M, l);  // groups [first, 1 + c(l-1)) hold this level's knots
        const bool elim = hasG && lev == l;
        if (__builtin_amdgcn_ballot_w64(elim) != 0) {
            chol_solve<NP, NC, KA>(e, i, bad, elim);  // other groups' rows stay as they are
            if (elim && rowi) {
#pragma unroll
                for (int c = 0; c < YW; ++c) sm.es[g - first][i][c] = e[NC + c];
            }
            if constexpr (REF) {
                if (elim && rowi) {
                    float r[16];
#pragma unroll
                    for (int c = 0; c < 16; ++c) r[c] = c < NC ? e[c] : 0.0f;
                    st4<16>(p.dws, ec_at(b, g) + 16 * ii, r);
                }
            }
        }
        __syncthreads();
        const bool kept = hasG && lev > l;
        if (__builtin_amdgcn_ballot_w64(kept) != 0) {
            const bool hasL = ke > 0, hasU = ke + s < N;
            const int gm = hasL ? cr_even_group((ke - s) / 2, M) - first : 0;
            const int gp = hasU ? cr_even_group((ke + s) / 2, M) - first : 0;
            update(kept, hasL, hasU, kept && lev == l + 1 && lev < levels, &sm.es[gm][0][0], &sm.es[gp][0][0]);
        }
        __syncthreads();
    }

    // last level: knot 0 alone (group 0); lambda now lives in LDS
    {
        const bool last = g == 0;
        if (__builtin_amdgcn_ballot_w64(last) != 0) {
            float a[NC + 1];
#pragma unroll
            for (int c = 0; c < NC; ++c) a[c] = e[c];
            a[NC] = e[3 * NC];
            chol_solve<NP, NC, NC + 1>(a, i, bad, last);
            if constexpr (REF) {
                if (last && rowi) {
                    float r[16];
#pragma unroll
                    for (int c = 0; c < 16; ++c) r[c] = c < NC ? a[c] : 0.0f;
                    st4<16>(p.dws, ec_at(b, 0) + 16 * ii, r);
                }
            }
            float dg = 1.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) dg = c == i ? a[c] : dg;
            float lam = 0.0f;
            tri_upper_solve<NP, NC>(a, a[NC], __builtin_amdgcn_rcpf(rowi ? dg : 1.0f), i, lam);
            nonfinite |= last && rowi && !__builtin_isfinite(lam);
            if (last && rowi) sm.lam[0][i] = lam;
        }
        __syncthreads();
    }

    // From here on, addresses and lane indices come from fresh copies of the
    // solve index and the thread index: what is formed from them above need not
    // stay live (or be spilled) until the back substitution and the recovery.
    int bl = late(b);
    auto refresh = [&]() {
        bl = late(b);
        const int tx = late_lane((int)threadIdx.x);
        i = tx % NP;
        g = tx / NP;
        rowi = i < NC;
        ii = rowi ? i : 0;
        hasG = g < M;
        jo = 2 * g + 1;
        hasO = hasG && jo < N;
        me = hasG ? cr_group_even(g, M) : 0;
        ke = 2 * me;
        lev = me == 0 ? levels : 1 + __builtin_ctz(me);
    };
    refresh();

    // back substitution, levels in reverse: lambda_j = C_j'^-1 (w3 - W1 lambda_{j-s} - W2 lambda_{j+s})
    auto back = [&](bool act, int k, int s, const float* ct, const float* w1, const float* w2, float w3) {
        const bool hasU = k + s < N;
        const float lm = (act && rowi) ? sm.lam[act ? k - s : 0][ii] : 0.0f;
        const float lp = (act && rowi && hasU) ? sm.lam[hasU ? k + s : 0][ii] : 0.0f;
        float acc = 0.0f;
        dotb<NP, NC>(acc, Bc<NP>(lm), w1);
        dotb<NP, NC>(acc, Bc<NP>(lp), w2);
        float dg = 1.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) dg = c == i ? ct[c] : dg;
        float lam = 0.0f;
        tri_upper_solve<NP, NC>(ct, w3 - acc, __builtin_amdgcn_rcpf((act && rowi) ? dg : 1.0f), i, lam);
        nonfinite |= act && rowi && !__builtin_isfinite(lam);
        if (act && rowi) sm.lam[k][i] = lam;
    };
    // every level's back substitution (the w3 of the even knots in e, of the odd knots in their LDS rows)
    auto back_sweep = [&]() {
        for (int l = levels - 1; l >= 1; --l) {
            const bool act = hasG && lev == l;
            if (__builtin_amdgcn_ballot_w64(act) != 0) back(act, ke, 1 << l, e, e + NC, e + 2 * NC, e[3 * NC]);
            __syncthreads();
        }
        if (levels >= 1) {
            if (__builtin_amdgcn_ballot_w64(hasO) != 0) {
                float w1[NC], w2[NC], oc[16];
                const size_t ocl =
                    VIRT ? nw.oc(bl, hasO ? g : 0, ii) : (((size_t)bl * M + (hasO ? g : 0)) * NC + ii) * 16;
                ld4<16>(p.dws, ocl, hasO && rowi, oc);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    w1[c] = sm.os[hasO ? g : 0][ii][c];
                    w2[c] = sm.os[hasO ? g : 0][ii][NC + c];
                }
                back(hasO, jo, 1, oc, w1, w2, sm.os[hasO ? g : 0][ii][2 * NC]);
            }
            __syncthreads();
        }
    };
    back_sweep();

    if constexpr (VIRT) {
        // lambda of the boundary knots, at their real positions
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const bool ok = w == 0 ? hasG : hasO;
            const int v = w == 0 ? ke : jo;
            if (ok && rowi) p.lambda[ix.vn(bl, nd_real(v, p.N), i)] = sm.lam[v][i];
        }
    } else if constexpr (!REF) {
        // recovery of this group's knots, and lambda to memory (both knots' loads issued together)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const bool ok = w == 0 ? hasG : hasO;
            if (__builtin_amdgcn_ballot_w64(ok) == 0) continue;
            const int kk = ok ? (w == 0 ? ke : jo) : 0;
            const bool rowv = ok && rowi;
            const float lam = rowv ? sm.lam[kk][ii] : 0.0f;
            const float lamn = (rowv && kk + 1 < N) ? sm.lam[kk + 1 < N ? kk + 1 : kk][ii] : 0.0f;
            if (rowv) p.lambda[ix.vn(bl, kk, i)] = lam;
            recover_knot<SH>(p, bl, kk, i, ok, lam, lamn);
        }
    } else {
        // ---- per knot: the first pass's dz (to memory, where the sums below add to
        // it, and to LDS), then the KKT residual (kkt_rows' q', r', e', x0', here
        // with the rows the recovery read kept for it) and the pieces of the
        // correction's gamma' as the formation forms gamma: h = Q~^-1 q',
        // t = A h + B R^-1 r'; e' less its dx_{k+1} term (in double) and t go to
        // LDS for knot k + 1.  q' and r' wait in the workspace, after the C' rows,
        // for the correction's recovery (this solve's rows from qpw and rpw on).
        refresh();
        float* const qpw = p.dws + 2 * ec0 + (size_t)bl * N * NC;
        float* const rpw = p.dws + 2 * ec0 + (size_t)p.B * N * NC + (size_t)bl * N * MC;
        float hh[2], gp[2];
        float x0p = 0.0f;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            mem_order();  // one knot's rows at a time
            const bool ok = w == 0 ? hasG : hasO;
            hh[w] = 0.0f;
            if (__builtin_amdgcn_ballot_w64(ok) == 0) continue;
            const int kk = ok ? (w == 0 ? ke : jo) : 0;
            // this knot's addresses from a fresh copy of the lane index (not kept for both knots)
            const int i = late_lane((int)threadIdx.x) % NP;
            const bool rowi = i < NC;
            const int ii = rowi ? i : 0;
            const bool rowv = ok && rowi, dyn = ok && kk < N - 1, urow = dyn && i < MC;
            const float lam = rowv ? sm.lam[kk][ii] : 0.0f;
            const float lamn = (rowv && kk + 1 < N) ? sm.lam[kk + 1 < N ? kk + 1 : kk][ii] : 0.0f;
            RecRows<SH> r;
            wave_prio<true, 3>();
            rec_load<SH>(p, bl, kk, i, ok, r);
            float dx, du;
            {
                float sup[NC];
                ld_row<NC>(p.S, ix.blk(bl, kk, 2, i), rowv, sup);
                float h = 0.0f;
                dotb<NP, NC>(h, Bc<NP>(r.qv), r.qi);
                recover<SH>(i, rowv, urow, lam, lamn, r.qi, sup, h, r.bc, r.rv, r.ri, dx, du);
            }
            wave_prio<true, 2>();
            float* const lamb = p.lambda + (size_t)bl * N * NC;  // this solve's lambda and dz
            float* const dzb = p.dz + ix.dx(bl, 0, 0);
            if (rowv) {
                sm.dx[kk][i] = dx;
                lamb[(unsigned)(kk * NC + i)] = lam;
                dzb[(unsigned)(kk * (NC + MC) + i)] = dx;
            }
            if (urow) {
                sm.du[kk][i] = du;
                dzb[(unsigned)(kk * (NC + MC) + NC + i)] = du;
            }
            __builtin_amdgcn_wave_barrier();  // the knot's dx and du, whole, for its own lanes
            seq_after(dx);
            const float* xv = sm.dx[kk];
            const float* uv = sm.du[kk];
            const float* lv = sm.lam[dyn ? kk + 1 : kk];
            // q'_k and r'_k (the terms of kkt_rows, in its order)
            double s = 0.0, sr = 0.0;
            {
                float qr[NC];
                ld_row<NC>(p.Q, ix.Q(bl, kk, i), rowv, qr);
                const double rh = p.rho != nullptr ? (double)p.rho[bl] : 0.0;
                s = (double)r.qv + rh * (rowv ? xv[ii] : 0.0f) - lam;
#pragma unroll
                for (int c = 0; c < NC; ++c) s += (double)qr[c] * xv[c];
            }
            seq_after(s);
            if (dyn) {
                float ac[NC];
                ld_row<NC, NC>(p.A, ix.A(bl, kk, 0) + i, rowi, ac);  // column i of A_k
#pragma unroll
                for (int c = 0; c < NC; ++c) s += (double)ac[c] * lv[c];
            }
            seq_after(s);
            {
                float rr[MC];
                ld_row<MC>(p.R, ix.R(bl, kk, i), urow, rr);
                sr = (double)r.rv;
#pragma unroll
                for (int c = 0; c < MC; ++c) sr += (double)rr[c] * uv[c];
#pragma unroll
                for (int c = 0; c < NC; ++c) sr += (double)r.bc[c] * lv[c];  // B_k' lambda_{k+1}
            }
            const float qv = rowv ? (float)s : 0.0f, rv = urow ? (float)sr : 0.0f;
            float h = 0.0f, gr = 0.0f;
            dotb<NP, NC>(h, Bc<NP>(qv), r.qi);
            dotb<NP, MC>(gr, Bc<NP>(rv), r.ri);
            h = rowv ? h : 0.0f;
            gr = urow ? gr : 0.0f;
            if (rowv) qpw[(unsigned)(kk * NC + i)] = qv;
            if (urow) rpw[(unsigned)(kk * MC + i)] = rv;
            seq_after(h);
            seq_after(gr);
            // e'_k without its -dx_{k+1} (double), t_k = A_k h + B_k R_k^-1 r'_k, and x0'
            {
                float ar[NC], br[MC];
                ld_row<NC>(p.A, ix.A(bl, kk, i), dyn && rowi, ar);
                ld_row<MC>(p.Bu, ix.Bu(bl, kk, i), dyn && rowi, br);
                const float ev = ld1(p.e, ix.e(bl, kk, i), dyn && rowi);
                double te = (double)ev;
#pragma unroll
                for (int c = 0; c < NC; ++c) te += (double)ar[c] * xv[c];
#pragma unroll
                for (int c = 0; c < MC; ++c) te += (double)br[c] * uv[c];
                float tt = 0.0f;
                dotb<NP, NC>(tt, Bc<NP>(h), ar);
                dotb<NP, MC>(tt, Bc<NP>(gr), br);
                if (dyn && rowi) {
                    sm.epd[kk][i] = te;
                    sm.ex[kk][i] = tt;
                }
                const float x0v = ld1(p.x0, (size_t)bl * NC + i, rowv && kk == 0);
                if (rowv && kk == 0) x0p = (float)((double)x0v - dx);
            }
            hh[w] = h;
        }
        wave_prio<true, 0>();
        __syncthreads();
        refresh();
        // gamma'_0 = x0' + h_0, gamma'_{k+1} = (e'_k - t_k) + h_{k+1}, e'_k = e_k + A dx_k + B du_k - dx_{k+1}
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const bool ok = w == 0 ? hasG : hasO;
            const int kk = ok ? (w == 0 ? ke : jo) : 0;
            const bool rowv = ok && rowi;
            const int km = kk > 0 ? kk - 1 : 0;
            const float ep = (float)(sm.epd[km][ii] - (double)sm.dx[kk][ii]);
            const float gx = (rowv && kk > 0) ? ep - sm.ex[km][ii] : x0p;
            gp[w] = rowv ? gx + hh[w] : 0.0f;
        }
        __syncthreads();  // the exchange rows are read before the second sweep reuses their LDS

        // ---- the second sweep: gamma' through the first pass's eliminations.
        // The kept knots' gamma' less W2m' w3m and W1p' w3p (rows of the
        // eliminated neighbours k - s and k + s, read by columns).
        auto gupdate = [&](bool kept, bool hasL, bool hasU, const float* Wm, const float* Wp) {
            const bool okm = kept && hasL && rowi, okp = kept && hasU && rowi;
            float s = 0.0f;
#pragma unroll
            for (int l = 0; l < NC; ++l) s = fmaf(okm ? Wm[l * YW + NC + ii] : 0.0f, okm ? Wm[l * YW + 2 * NC] : 0.0f, s);
#pragma unroll
            for (int l = 0; l < NC; ++l) s = fmaf(okp ? Wp[l * YW + ii] : 0.0f, okp ? Wp[l * YW + 2 * NC] : 0.0f, s);
            if (kept && rowi) e[3 * NC] -= s;
        };
        refresh();
        e[3 * NC] = hasG ? gp[0] : 0.0f;
        // the factors back in registers: the even knot's C' rows (the last Schur
        // complement's for knot 0), and the odd knot's C' by columns (row i of C)
        float cl[NC];
        {
            float ct[16];
            ld4<16>(p.dws, ec_at(bl, hasG ? g : 0) + 16 * ii, hasG && rowi, ct);
#pragma unroll
            for (int c = 0; c < NC; ++c) e[c] = ct[c];
            ld_row<NC, 16>(p.dws, ((size_t)bl * M + (hasO ? g : 0)) * NC * 16 + ii, hasO && rowi, cl);
        }
        // level 0: the odd knots
        if (__builtin_amdgcn_ballot_w64(hasO) != 0) {
            float dg = 1.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) dg = c == i ? cl[c] : dg;
            float w3 = 0.0f;
            tri_lower_solve<NP, NC>(cl, (hasO && rowi) ? gp[1] : 0.0f,
                                    __builtin_amdgcn_rcpf((hasO && rowi) ? dg : 1.0f), i, w3);
            if (hasO && rowi) sm.os[g][i][2 * NC] = w3;
        }
        __syncthreads();
        if (__builtin_amdgcn_ballot_w64(hasG) != 0) {
            const bool hasL = ke > 0, hasU = ke + 1 < N;
            gupdate(hasG, hasL, hasU, &sm.os[hasL ? me - 1 : 0][0][0], &sm.os[hasU ? me : 0][0][0]);
        }
        __syncthreads();
        // levels 1 .. levels-1: w3' with C by columns, then the W rows to the level's slot
        for (int l = 1; l < levels; ++l) {
            const int s = 1 << l;
            const int first = 1 + cr_mult(M, l);
            const bool elim = hasG && lev == l;
            if (__builtin_amdgcn_ballot_w64(elim) != 0) {
                // C' through the knot's own slot of the level (one wave): row i of C back
                float* slot = &sm.es[elim ? g - first : 0][0][0];
                if (elim && rowi)
#pragma unroll
                    for (int c = 0; c < NC; ++c) slot[i * YW + c] = e[c];
                __builtin_amdgcn_wave_barrier();
                float cc[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) cc[c] = (elim && rowi) ? slot[c * YW + ii] : 0.0f;
                __builtin_amdgcn_wave_barrier();
                float dg = 1.0f;
#pragma unroll
                for (int c = 0; c < NC; ++c) dg = c == i ? e[c] : dg;
                float w3 = 0.0f;
                tri_lower_solve<NP, NC>(cc, (elim && rowi) ? e[3 * NC] : 0.0f,
                                        __builtin_amdgcn_rcpf((elim && rowi) ? dg : 1.0f), i, w3);
                e[3 * NC] = elim ? w3 : e[3 * NC];
                if (elim && rowi)
#pragma unroll
                    for (int c = 0; c < YW; ++c) slot[i * YW + c] = e[NC + c];
            }
            __syncthreads();
            const bool kept = hasG && lev > l;
            if (__builtin_amdgcn_ballot_w64(kept) != 0) {
                const bool hasL = ke > 0, hasU = ke + s < N;
                const int gm = hasL ? cr_even_group((ke - s) / 2, M) - first : 0;
                const int gq = hasU ? cr_even_group((ke + s) / 2, M) - first : 0;
                gupdate(kept, hasL, hasU, &sm.es[gm][0][0], &sm.es[gq][0][0]);
            }
            __syncthreads();
        }
        // last level: knot 0, with the factor of its last Schur complement
        {
            const bool last = g == 0;
            if (__builtin_amdgcn_ballot_w64(last) != 0) {
                float* slot = &sm.es[0][0][0];
                if (last && rowi)
#pragma unroll
                    for (int c = 0; c < NC; ++c) slot[i * YW + c] = e[c];
                __builtin_amdgcn_wave_barrier();
                float cc[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) cc[c] = (last && rowi) ? slot[c * YW + ii] : 0.0f;
                __builtin_amdgcn_wave_barrier();
                float dg = 1.0f;
#pragma unroll
                for (int c = 0; c < NC; ++c) dg = c == i ? e[c] : dg;
                const float dinv = __builtin_amdgcn_rcpf((last && rowi) ? dg : 1.0f);
                float w3 = 0.0f, lam = 0.0f;
                tri_lower_solve<NP, NC>(cc, (last && rowi) ? e[3 * NC] : 0.0f, dinv, i, w3);
                tri_upper_solve<NP, NC>(e, w3, dinv, i, lam);
                nonfinite |= last && rowi && !__builtin_isfinite(lam);
                if (last && rowi) sm.lam[0][i] = lam;
            }
            __syncthreads();
        }
        refresh();
        back_sweep();

        // ---- the correction's dz (its q' and r', h = Q~^-1 q' as above), and the sums
        // (both knots' loads issued together)
        refresh();
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const bool ok = w == 0 ? hasG : hasO;
            if (__builtin_amdgcn_ballot_w64(ok) == 0) continue;
            const int kk = ok ? (w == 0 ? ke : jo) : 0;
            const bool rowv = ok && rowi, urow = ok && kk < N - 1 && i < MC;
            const float mu = rowv ? sm.lam[kk][ii] : 0.0f;
            const float mun = (rowv && kk + 1 < N) ? sm.lam[kk + 1 < N ? kk + 1 : kk][ii] : 0.0f;
            float qi[NC], ri[MC], bc[NC], sup[NC];
            wave_prio<true, 3>();
            ld_row<NC>(p.Qinv, ix.Q(bl, kk, i), rowv, qi);
            ld_row<MC>(p.Rinv, ix.R(bl, kk, i), urow, ri);
            ld_row<NC, MC>(p.Bu, ix.Bu(bl, kk, 0) + i, urow, bc);  // column i of B_k
            ld_row<NC>(p.S, ix.blk(bl, kk, 2, i), rowv, sup);
            const float qv = ld1(qpw, (unsigned)(kk * NC + i), rowv);
            const float rv = ld1(rpw, (unsigned)(kk * MC + i), urow);
            float h = 0.0f;  // (Q~_k^-1 q'_k)_i, as above
            dotb<NP, NC>(h, Bc<NP>(qv), qi);
            float ddx, ddu;
            recover<SH>(i, rowv, urow, mu, mun, qi, sup, h, bc, rv, ri, ddx, ddu);
            float* const lamb = p.lambda + (size_t)bl * N * NC;  // this solve's lambda and dz
            float* const dzb = p.dz + ix.dx(bl, 0, 0);
            if (rowv) {
                lamb[(unsigned)(kk * NC + i)] += mu;
                dzb[(unsigned)(kk * (NC + MC) + i)] += ddx;
            }
            if (urow) dzb[(unsigned)(kk * (NC + MC) + NC + i)] += ddu;
            wave_prio<true, 1>();
        }
        wave_prio<true, 0>();
    }

    const int fl = (bad ? GATO_F_S_NOT_SPD : 0) | (nonfinite ? GATO_F_NONFINITE : 0);
    if (fl) atomicOr(&sm.flags, fl);
    __syncthreads();
    if (threadIdx.x == 0) {
        p.flags[bl] |= sm.flags;
        if (p.iters) p.iters[bl] = 0;
        if (p.relres) p.relres[bl] = 0.0f;
    }
}

// ------------------------------------------------------------------ nested dissection, chunk interiors

template <class SH>
struct NdLds {
    float t[ND_GPW][SH::NC][SH::NC + 1];  // one transpose tile per lane group (+1: bank spread)
    int flags;
};

// Eliminates every chunk's interior knots in order (lane group g: chunk g).
// The chunk's first knot a stays in registers and collects the Schur
// complement of the knots eliminated so far, together with its coupling F to
// the current front knot f; eliminating f (D_f = C C', W1 = C^-1 F', W2 =
// C^-1 U_f, w3 = C^-1 gamma_f) updates
//   D_a -= W1'W1, gamma_a -= W1'w3, F <- -W1'W2 (now the coupling a <-> f+1),
//   D_{f+1} -= W2'W2, gamma_{f+1} -= W2'w3.
// Each front's factor (W1, w3 and C') goes to the workspace for the back substitution.
// Afterwards the chunk's first and last knots, with F between them and S's own
// coupling to the next chunk, are rows of the boundary system.  Transposes go
// through the group's own LDS tile (no barrier: the tile belongs to one wave).
template <class SH>
__device__ __forceinline__ void nd_reduce(const Params& p, int b)
{
    constexpr int NP = SH::NP, NC = SH::NC;
    static_assert(NP == 16, "one knot row per lane of a 16-lane group");
    constexpr int KA = 3 * NC + 1;
    using RW = CrRow<SH>;
    constexpr int W = RW::W;
    __shared__ NdLds<SH> sm;
    const Ix<SH> ix{p.N};
    const NdWs<SH> nw{(size_t)p.B, (size_t)p.N};
    const int N = p.N;
    const int i = threadIdx.x % NP;
    const int g = blockIdx.y * ND_GPW + threadIdx.x / NP;  // chunk
    const bool rowi = i < NC;
    const int ii = rowi ? i : 0;
    const int a = nd_start(g, N), bk = nd_start(g + 1, N) - 1;
    const int nint = bk - a - 1;  // interior knots (chunks hold >= 2 knots)
    const int maxint = (N + ND_CHUNKS - 1) / ND_CHUNKS - 2;
    float(*t)[NC + 1] = sm.t[threadIdx.x / NP];
    if (threadIdx.x == 0) sm.flags = 0;
    __syncthreads();  // the flag word is zero before any wave can set a bit in it
    bool bad = false;

    auto transpose = [&](const float* x, float* out) {  // out[c] = X[c][i], X's row i in lane i
        if (rowi) {
#pragma unroll
            for (int c = 0; c < NC; ++c) t[i][c] = x[c];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int c = 0; c < NC; ++c) out[c] = t[c][ii];
        __builtin_amdgcn_wave_barrier();
    };

    float Da[NC], F[NC], Dn[NC];
    ld_row<NC>(p.S, ix.blk(b, a, 1, i), rowi, Da);
    ld_row<NC>(p.S, ix.blk(b, a, 2, i), rowi, F);  // coupling a <-> a+1
    ld_row<NC>(p.S, ix.blk(b, a + 1, 1, i), rowi, Dn);
    float ga = ld1(p.gamma, ix.vn(b, a, i), rowi);
    float gn = ld1(p.gamma, ix.vn(b, a + 1, i), rowi);

    // One elimination step on front f, given U_f (its coupling to f + 1) and
    // D_{f+1}, gamma_{f+1} as loaded; groups with act false (their chunk has one
    // interior knot fewer) run it with zero multipliers and keep their state.
    auto step = [&](int f, bool act, const float* Uf, const float* Dx, float gx) {
        float x[KA];  // [D_f | F' | U_f | gamma_f]
#pragma unroll
        for (int c = 0; c < NC; ++c) x[2 * NC + c] = Uf[c];
        transpose(F, x + NC);
#pragma unroll
        for (int c = 0; c < NC; ++c) x[c] = Dn[c];
        x[3 * NC] = gn;
        chol_solve<NP, NC, KA>(x, i, bad, act);
        if (act && rowi) {  // the factor: row i of [W1 | w3], then row i of C' from its diagonal on
            constexpr int R1 = NdWs<SH>::R1;
            float r[R1];
#pragma unroll
            for (int c = 0; c < R1; ++c) r[c] = c < NC ? x[NC + c] : 0.0f;
            r[NC] = x[3 * NC];
            st4<R1>(p.dws, nw.fac(b, f, i), r);
            float* ct = p.dws + nw.tri(b, f) + (nd_tri_off(i, NC) - i);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                if (c >= i) ct[c] = x[c];
        }
        if constexpr (SH::MMA && NC < 16) {
            // (columns)' (columns) on the matrix cores: lane c holds column c
            // of W1 (then W2), and lane n the column w3, so each sum's column n
            // is the gamma update.  Groups with act false get zero products.
            auto columns = [&](const float* w, float* out) {  // out[k] = W[k][lane], w3 at lane n
                if (rowi) {
#pragma unroll
                    for (int c = 0; c < NC; ++c) t[i][c] = w[c];
                    t[i][NC] = x[3 * NC];
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int k = 0; k < NC; ++k) out[k] = (act && i <= NC) ? t[k][i <= NC ? i : 0] : 0.0f;
                __builtin_amdgcn_wave_barrier();
            };
            float w1[NC], w2[NC], r[NC + 1];
            columns(x + NC, w1);
            columns(x + 2 * NC, w2);
            // the chunk's first knot: D_a -= W1' W1, gamma_a -= W1' w3, F = -W1' W2
            mma16_t acc = {};
            mma_abt<NC>(acc, w1, w1);
            mma_rows<NC + 1>(acc, r);
#pragma unroll
            for (int k = 0; k < NC; ++k) Da[k] = rowi ? Da[k] - r[k] : Da[k];
            ga = rowi ? ga - r[NC] : ga;
            acc = mma16_t{};
            mma_abt<NC>(acc, w1, w2);
            mma_rows<NC>(acc, r);
#pragma unroll
            for (int k = 0; k < NC; ++k) F[k] = act ? (rowi ? 0.0f - r[k] : 0.0f) : F[k];
            // the next front: D_{f+1} -= W2' W2, gamma_{f+1} -= W2' w3
            acc = mma16_t{};
            mma_abt<NC>(acc, w2, w2);
            mma_rows<NC + 1>(acc, r);
#pragma unroll
            for (int k = 0; k < NC; ++k) Dn[k] = act ? (rowi ? Dx[k] - r[k] : Dx[k]) : Dn[k];
            gn = act ? (rowi ? gx - r[NC] : gx) : gn;
            return;
        }
        float c[NC];  // -(column i of W1), then -(column i of W2)
        transpose(x + NC, c);
#pragma unroll
        for (int k = 0; k < NC; ++k) c[k] = (act && rowi) ? -c[k] : 0.0f;
        // the chunk's first knot; the old F is no longer needed (W1 carries it)
        gemm_rows<NP, NC, NC>(Da, BcRow<NP, NC>(x + NC), c);
        dotb<NP, NC>(ga, Bc<NP>(x[3 * NC]), c);
#pragma unroll
        for (int k = 0; k < NC; ++k) F[k] = act ? 0.0f : F[k];
        gemm_rows<NP, NC, NC>(F, BcRow<NP, NC>(x + 2 * NC), c);
        // the next front (groups that are done keep their last knot's rows)
        transpose(x + 2 * NC, c);
        {
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                c[k] = (act && rowi) ? -c[k] : 0.0f;
                Dn[k] = act ? Dx[k] : Dn[k];
            }
            gn = act ? gx : gn;
        }
        gemm_rows<NP, NC, NC>(Dn, BcRow<NP, NC>(x + 2 * NC), c);
        dotb<NP, NC>(gn, Bc<NP>(x[3 * NC]), c);
    };

    // The steps every chunk has, then the one that the longer chunks have in
    // addition; each step's rows are requested one step ahead, so that their
    // latency overlaps the previous step's arithmetic.
    const int minint = N / ND_CHUNKS - 2;
    auto fetch = [&](int st, float* U, float* D, float& gv) {  // U_f, D_{f+1}, gamma_{f+1} of step st
        const bool ok = st < nint && rowi;
        const int f = ok ? a + 1 + st : a;
        ld_row<NC>(p.S, ix.blk(b, f, 2, i), ok, U);
        ld_row<NC>(p.S, ix.blk(b, f + 1, 1, i), ok, D);
        gv = ld1(p.gamma, ix.vn(b, f + 1, i), ok);
    };
    float Uc[NC], Dc[NC], gc;
    fetch(0, Uc, Dc, gc);
    for (int st = 0; st < maxint; ++st) {
        float Un[NC], Dnx[NC], gnx;
        fetch(st + 1, Un, Dnx, gnx);
        if (st < minint) {
            step(a + 1 + st, true, Uc, Dc, gc);
        } else {
            const bool act = nint > minint;
            step(act ? a + 1 + st : a + 1, act, Uc, Dc, gc);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            Uc[c] = Un[c];
            Dc[c] = Dnx[c];
        }
        gc = gnx;
    }

    // rows of the boundary system: knot 2g (= a): [- | F | gamma_a | D_a];
    // knot 2g+1 (= bk): [F' | S_{bk,bk+1} | gamma_bk | D_bk]
    float Lb[NC], Ub[NC];
    transpose(F, Lb);
    ld_row<NC>(p.S, ix.blk(b, bk, 2, i), rowi && bk + 1 < N, Ub);
    if (rowi) {
        float r[W];
#pragma unroll
        for (int c = 0; c < W; ++c) r[c] = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            r[RW::U + c] = F[c];
            r[RW::D + c] = Da[c];
        }
        r[RW::G] = ga;
        st4<W>(p.dws, nw.vrow(b, 2 * g, i), r);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            r[RW::L + c] = Lb[c];
            r[RW::U + c] = Ub[c];
            r[RW::D + c] = Dn[c];
        }
        r[RW::G] = gn;
        st4<W>(p.dws, nw.vrow(b, 2 * g + 1, i), r);
    }
    if (bad) atomicOr(&sm.flags, GATO_F_S_NOT_SPD);
    __syncthreads();
    if (threadIdx.x == 0 && sm.flags) atomicOr(p.flags + b, sm.flags);  // the solve's other workgroups too
}

// Back substitution of every chunk's interior knots (the chunk's first and last
// knots have lambda from the boundary system), last interior knot first:
//   lambda_f = C_f'^-1 (w3_f - W1_f lambda_a - C_f^-1 U_f lambda_{f+1}),
// with the recovery of dz for every knot of the chunk by the same lane group:
// the last knot first, then each interior knot as soon as its lambda is known
// (U_f = S_{f,f+1} is then still in registers), the first knot last.
template <class SH>
__device__ __forceinline__ void nd_back(const Params& p, int b)
{
    constexpr int NP = SH::NP, NC = SH::NC;
    constexpr int R1 = NdWs<SH>::R1;
    __shared__ int wg_flags;
    const Ix<SH> ix{p.N};
    const NdWs<SH> nw{(size_t)p.B, (size_t)p.N};
    const int N = p.N;
    const int i = threadIdx.x % NP;
    const int g = blockIdx.y * ND_GPW + threadIdx.x / NP;  // chunk
    const bool rowi = i < NC;
    const int ii = rowi ? i : 0;
    const int a = nd_start(g, N), bk = nd_start(g + 1, N) - 1;
    const int maxint = (N + ND_CHUNKS - 1) / ND_CHUNKS - 2;
    if (threadIdx.x == 0) wg_flags = 0;
    __syncthreads();  // the flag word is zero before any wave can set a bit in it
    bool nonfinite = false;

    // What lane i needs of interior knot k: row i of [W1 | w3], row i of C' and
    // column i of C' (both from the packed triangle, zero off it), row i of
    // U_k = S_{k,k+1}, and the rest of the knot's recovery rows.  ok false
    // reads zeros; k must still be a knot of the solve, and every index stays
    // inside that knot's factor.
    struct Fac {
        float w[R1], row[NC], col[NC], u[NC];
        RecRows<SH> rec;
    };
    auto fetch = [&](int k, bool ok, Fac& f) {
        ld4<R1>(p.dws, nw.fac(b, k, ii), ok, f.w);
        const float* t = p.dws + nw.tri(b, k);
        const float* tr = t + (nd_tri_off(ii, NC) - ii);  // C'[i][c] at tr[c] for c >= i
        const float* tc = t + ii;                         // C'[c][i] at tc[off(c) - c] for c <= i
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            f.row[c] = (ok && c >= i) ? tr[c] : 0.0f;
            f.col[c] = (ok && c <= i) ? tc[nd_tri_off(c, NC) - c] : 0.0f;
        }
        ld_row<NC>(p.S, ix.blk(b, k, 2, ii), ok, f.u);
        rec_load<SH>(p, b, k, i, ok, f.rec);
    };

    const float la = ld1(p.lambda, ix.vn(b, a, i), rowi);
    float lamn = ld1(p.lambda, ix.vn(b, bk, i), rowi);  // lambda of the knot after the front
    Fac cur;
    fetch(bk - 1 > a ? bk - 1 : a, rowi && bk - 1 > a, cur);
    {
        // the chunk's last knot: lambda_{bk+1} is the next chunk's first knot's
        const float lnx = ld1(p.lambda, ix.vn(b, bk + 1 < N ? bk + 1 : bk, i), rowi && bk + 1 < N);
        recover_knot<SH>(p, b, bk, i, true, lamn, lnx);
    }
    for (int st = 0; st < maxint; ++st) {
        const int k = bk - 1 - st;
        const bool act = k > a;
        if (__builtin_amdgcn_ballot_w64(act) == 0) continue;
        Fac nxt;
        fetch(k - 1 > a ? k - 1 : a, rowi && k - 1 > a, nxt);
        float v = 0.0f;  // W1 lambda_a
        dotb<NP, NC>(v, Bc<NP>(la), cur.w);
        float u = 0.0f;  // U_k lambda_{k+1}
        dotb<NP, NC>(u, Bc<NP>(lamn), cur.u);
        float dg = 1.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) dg = c == i ? cur.row[c] : dg;
        const float dinv = __builtin_amdgcn_rcpf((act && rowi) ? dg : 1.0f);
        float y = 0.0f;  // C^-1 U_k lambda_{k+1}, the W2 term
        tri_lower_solve<NP, NC>(cur.col, u, dinv, i, y);
        float lin = 0.0f;
        tri_upper_solve<NP, NC>(cur.row, cur.w[NC] - v - y, dinv, i, lin);
        nonfinite |= act && rowi && !__builtin_isfinite(lin);
        if (act && rowi) p.lambda[ix.vn(b, k, i)] = lin;
        rec_store<SH>(p, b, k, i, act, cur.rec, cur.u, lin, lamn);
        lamn = act ? lin : lamn;
        cur = nxt;
    }
    recover_knot<SH>(p, b, a, i, true, la, lamn);  // the chunk's first knot
    if (nonfinite) atomicOr(&wg_flags, GATO_F_NONFINITE);
    __syncthreads();
    if (threadIdx.x == 0 && wg_flags) atomicOr(p.flags + b, wg_flags);
}

}  // namespace gato
