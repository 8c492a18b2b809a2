// gato_stages.h -- the three stages of the SQP-step core as workgroup-level
// device functions (GATO paper, Sec. II-III).  Every function is called by all
// threads of a workgroup in uniform control flow; lane (slot s, row i) holds
// row i of knot w0 + s.  Shapes are compile-time (n = NC, m = MC), so all
// index arithmetic folds into immediate offsets; loads that may fall outside
// the problem read a valid dummy address and are masked afterwards, so no
// load sits behind a branch.
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
    int s_upper_only;  // stage 1 alone: write S's diagonal and upper blocks only (the solve reads no lower block)
    int cr_stream;     // cyclic reduction: the streaming kernel (every level's rows in the workspace) for any n
    float* dws;   // direct solve: pivot inverses [B][N][n][n], then eliminated right-hand sides [B][N][n]
    float* mpart;  // merit split over workgroups: per-knot values [B][n_alpha + 1][N]
};

// The same value in every lane (the reductions below produce identical bits in
// all lanes); moving it to a scalar register lets branches on it be scalar.
// Materialise x in a register here, so that a load feeding it is issued and
// waited for at this point rather than sunk past a later branch.
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }

// An opaque copy of a uniform index: addresses formed from it after this point
// are recomputed there instead of being kept live (or spilled) from an earlier
// computation of the same expression.
__device__ __forceinline__ int late(int x)
{
    asm volatile("" : "+s"(x));
    return x;
}

// The same for a per-lane value (a thread index): indices and addresses formed
// from the copy are recomputed where they are used.
__device__ __forceinline__ int late_lane(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// No memory access moves across this point: the loads after it are issued
// after what comes before has used its own, so the rows of two phases are not
// live at once.
__device__ __forceinline__ void mem_order() { asm volatile("" ::: "memory"); }

// x is formed before this point and no memory access moves across it: the
// loads x needs are consumed here, before any later load is issued.
__device__ __forceinline__ void seq_after(float x) { asm volatile("" ::"v"(x) : "memory"); }
__device__ __forceinline__ void seq_after(double x) { asm volatile("" ::"v"(x) : "memory"); }

__device__ __forceinline__ int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Float tests on the bit patterns, so that for values in scalar registers they
// are scalar integer instructions (no round trip through the vector unit):
// finite <=> the exponent is not all ones; for non-negative, non-NaN x and y,
// x <= y <=> bits(x) <= bits(y); x > 0 <=> bits(x) > 0 as a signed integer
// (for x not NaN).
__device__ __forceinline__ bool finite_bits(float x) { return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u; }
__device__ __forceinline__ bool le_nonneg_bits(float x, float y) { return __float_as_uint(x) <= __float_as_uint(y); }
__device__ __forceinline__ bool pos_bits(float x) { return __float_as_int(x) > 0; }

// This wave's issue priority (0 lowest .. 3), when ON.  The phases between
// two barriers step it down as they go (3 at the start, lower for later
// stages), so that the waves of a SIMD that are behind, which are the younger
// ones when the priorities are equal, issue first and the four reach the
// barrier closer together, with less of the phase left to one wave alone.
template <bool ON = true, int K = 0>
__device__ __forceinline__ void wave_prio()
{
    if constexpr (ON) __builtin_amdgcn_s_setprio(K);
}

__device__ __forceinline__ float uniform(float x)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// A flag taken through a wave ballot right where it is computed: the ballot
// is convergent and cannot be moved, so the pivot tests it depends on run in
// place instead of keeping every pivot alive until the flag is finally read.
__device__ __forceinline__ bool lane_bit(uint64_t mask)
{
    return (mask >> (threadIdx.x & 63)) & 1u;
}

// Whether any lane of this lane's group of NP has its bit set in mask.
template <int NP>
__device__ __forceinline__ bool group_any(uint64_t mask)
{
    const int sh = (threadIdx.x & 63) & ~(NP - 1);
    const uint64_t g = NP == 64 ? ~0ull : ((1ull << NP) - 1);
    return ((mask >> sh) & g) != 0;
}

// ------------------------------------------------------------------ indexing

template <class SH>
struct Ix {
    static constexpr int n = SH::NC, m = SH::MC;
    int N;
    __device__ __forceinline__ size_t kn(int b, int k) const { return (size_t)b * N + k; }
    __device__ __forceinline__ size_t kd(int b, int k) const { return (size_t)b * (N - 1) + k; }
    __device__ __forceinline__ size_t Q(int b, int k, int i) const { return (kn(b, k) * n + i) * n; }
    __device__ __forceinline__ size_t vn(int b, int k, int i) const { return kn(b, k) * n + i; }
    __device__ __forceinline__ size_t R(int b, int k, int i) const { return (kd(b, k) * m + i) * m; }
    __device__ __forceinline__ size_t vm(int b, int k, int i) const { return kd(b, k) * m + i; }
    __device__ __forceinline__ size_t A(int b, int k, int i) const { return (kd(b, k) * n + i) * n; }
    __device__ __forceinline__ size_t Bu(int b, int k, int i) const { return (kd(b, k) * n + i) * m; }
    __device__ __forceinline__ size_t e(int b, int k, int i) const { return kd(b, k) * n + i; }
    __device__ __forceinline__ size_t blk(int b, int k, int s, int i) const { return ((kn(b, k) * 3 + s) * n + i) * n; }
    __device__ __forceinline__ size_t nz() const { return (size_t)N * n + (size_t)(N - 1) * m; }
    __device__ __forceinline__ size_t dx(int b, int k, int i) const { return (size_t)b * nz() + (size_t)k * (n + m) + i; }
    __device__ __forceinline__ size_t du(int b, int k, int i) const
    {
        return (size_t)b * nz() + (size_t)k * (n + m) + n + i;
    }
};

// Masked loads read this page instead of the problem arrays, which may be
// absent in a call (NULL) or empty (N = 1).  4096 floats cover the widest
// strided read (a column of the cyclic reduction's 28 x 88 workspace rows);
// module globals are zero-initialised.
static __device__ __align__(16) float g_zero_page[4096];

// Load K floats at base[off + j * STRIDE] when ok, else zeros; the address is
// selected before the loads, which are then unconditional.
template <int K, int STRIDE = 1>
__device__ __forceinline__ void ld_row(const float* base, size_t off, bool ok, float* out)
{
    static_assert((K - 1) * STRIDE < 4096, "masked row read exceeds the zero page");
    const float* a = ok ? base + off : g_zero_page;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const float v = a[j * STRIDE];
        out[j] = ok ? v : 0.0f;
    }
}

__device__ __forceinline__ float ld1(const float* base, size_t off, bool ok)
{
    const float v = *(ok ? base + off : g_zero_page);
    return ok ? v : 0.0f;
}

// Rows of one knot's block rows of S and Phi^-1, and gamma, held by lane i.
template <class SH>
struct Rows {
    float slo[SH::NC], sd[SH::NC], sup[SH::NC];
    float plo[SH::NC], pd[SH::NC], pup[SH::NC];
    float gam;
};

// LDS the formation needs only while it runs (reusable afterwards) ...
template <class SH>
struct FormLds {
    float xw[SH::SLOTS][SH::NP][SH::NC + 1];  // one matrix row per lane (+1: bank spread)
    float xg[SH::SLOTS][SH::NP];
    alignas(16) float piv[SH::NP == 32 ? SH::SLOTS : 1][GJ_LDS_BLOCK * ((SH::NC + 3) / 4 * 4)];  // pivot rows (32-lane groups)
};

// In-place inverse of the K x K SPD matrix whose row i is held by lane i of
// group s: DPP broadcasts for 16-lane groups, the group's LDS row buffer for
// 32-lane ones.
template <class SH, int K>
__device__ __forceinline__ void inv_rows(float* a, int i, bool& bad, FormLds<SH>& L, int s)
{
    if constexpr (SH::NP == 32) gj_steps_lds<K>(a, i, bad, L.piv[s]);
    else gj_steps<SH::NP, K>(a, i, bad);
}

// ... and what it parks, which the fused step keeps for the recovery.
template <class SH>
struct Park {
    float Q[SH::SLOTS][SH::NC][SH::NC];   // Q~_k^-1 rows
    float R[SH::SLOTS][SH::MC][SH::MC];   // R_k^-1 rows
    float Bt[SH::SLOTS][SH::MC][SH::NC];  // B_k columns (rows of B_k')
    float h[SH::SLOTS][SH::NP];           // Q~_k^-1 q_k
    float rv[SH::SLOTS][SH::NP];          // r_k
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
// Q~_k^-1 and R_k^-1 rows, B_k's columns, Q~_k^-1 q_k and r_k are parked in
// LDS (K; the fused step keeps them for the recovery, the standalone kernel
// stores the inverses from there); the inverse rows are also handed to `sink`.
// `fl` gets the Q/R/S_NOT_SPD bits of this knot.  With PRE false the stair
// preconditioner (D_k^-1 and the Phi^-1 rows) is not formed: the direct solve
// does not use it, and S_NOT_SPD then comes from the solve's own pivots.
// PRIO: stage-ordered wave priorities (wave_prio), for one workgroup per CU;
// with the windowed formation's two workgroups per CU they cost time.
template <class SH, bool PRE = true, bool PRIO = false, class Sink>
__device__ __forceinline__ void form(const Params& p, int b, int w0, int nslot, FormLds<SH>& L, Park<SH>& K,
                                     Rows<SH>& out, int& fl, Sink sink)
{
    constexpr int NC = SH::NC, MC = SH::MC, NP = SH::NP, SL = SH::SLOTS;
    const Ix<SH> ix{p.N};
    const int N = p.N;
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    const int k = w0 + s;
    const bool kv = s < nslot && k < N;
    const bool hn = kv && k < N - 1;
    const bool rowv = kv && i < NC;
    const bool urow = hn && i < MC;
    const float rh = (p.rho != nullptr) ? p.rho[b] : 0.0f;
    const int sp = s > 0 ? s - 1 : 0;  // previous slot (clamped)
    const bool has_prev = s >= 1 && k >= 1;

    // The rows the inversions need first; the rows for the products are requested
    // after the first inversion (below), so that a wave is not held at its start
    // until all of its loads are accepted, and they arrive during the second.
    float qi0[NC], ri0[MC], ar[NC], br[MC];
    float qv, rv, ev;
    ld_row<NC>(p.Q, ix.Q(b, k, i), rowv, qi0);
    ld_row<MC>(p.R, ix.R(b, k, i), urow, ri0);

    // (wave priorities by stage: wave_prio)
    wave_prio<PRIO, 3>();
    // Q~_k^-1 (identity rows on lanes/knots outside the problem keep it finite)
    bool badq = false, badr = false, bads = false;
    {
        float qi[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) qi[c] = qi0[c];
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (c == i) qi[c] = rowv ? qi[c] + rh : 1.0f;
        inv_rows<SH, NC>(qi, i, badq, L, s);
        ld_row<NC>(p.A, ix.A(b, k, i), hn && i < NC, ar);
        ld_row<MC>(p.Bu, ix.Bu(b, k, i), hn && i < NC, br);
        qv = ld1(p.q, ix.vn(b, k, i), rowv);
        rv = ld1(p.r, ix.vm(b, k, i), urow);
        ev = ld1(p.e, ix.e(b, k, i), hn && i < NC);
        wave_prio<PRIO, 2>();
        badq = group_any<SH::NP>(__builtin_amdgcn_ballot_w64(badq));
        if (i < NC)
#pragma unroll
            for (int c = 0; c < NC; ++c) K.Q[s][i][c] = qi[c];
        float ri[MC];
#pragma unroll
        for (int c = 0; c < MC; ++c) ri[c] = (c == i) ? (urow ? ri0[c] : 1.0f) : ri0[c];
        inv_rows<SH, MC>(ri, i, badr, L, s);
        wave_prio<PRIO, 1>();
        badr = group_any<SH::NP>(__builtin_amdgcn_ballot_w64(badr));
        if (i < MC)
#pragma unroll
            for (int c = 0; c < MC; ++c) K.R[s][i][c] = ri[c];
        sink(qi, ri);
    }

    // W = A_k Q~_k^-1 (row i), V = B_k R_k^-1 (row i); gamma pieces
    //   h = (Q~_k^-1 q_k)_i (own knot), g = (e_k - W q_k - V r_k)_i (for knot k+1)
    // On the matrix cores U_k = W_k A_k' + V_k B_k' is formed here too, while
    // W_k's rows are still in registers (the DPP form below takes O_k's rows).
    float V[MC], h = 0.0f, g;
    float U[NC];
    {
        float qi[NC], ri[MC], W[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) qi[c] = K.Q[s][i < NC ? i : 0][c];
#pragma unroll
        for (int c = 0; c < MC; ++c) ri[c] = K.R[s][i < MC ? i : 0][c];
        if (i < NC)
#pragma unroll
            for (int c = 0; c < MC; ++c) K.Bt[s][c][i] = br[c];  // transpose of B_k
#pragma unroll
        for (int c = 0; c < MC; ++c) V[c] = 0.0f;
        if constexpr (SH::MMA) {
            mma_t<NP> acc = {};
            mma_abt<NC>(acc, ar, qi);  // A_k Q~_k^-1' (Q~_k^-1 is symmetric)
            mma_rows<NC>(acc, W);
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) W[c] = 0.0f;
            gemm_rows<NP, NC, NC>(W, BcRow<NP, NC>(qi), ar);
        }
        gemm_rows<NP, MC, MC>(V, BcRow<NP, MC>(ri), br);
        if constexpr (SH::MMA) {
            mma_t<NP> acc = {};
            mma_abt<NC>(acc, ar, W);  // A_k W_k' = A_k Q~_k^-1 A_k'
            mma_abt<MC>(acc, V, br);  // V_k B_k' = B_k R_k^-1 B_k'
            mma_rows<NC>(acc, U);
        }
        float t1 = 0.0f, t2 = 0.0f;
        const Bc<NP> qb(qv);
        dotb<NP, NC>(h, qb, qi);
        dotb<NP, NC>(t1, qb, W);
        dotb<NP, MC>(t2, Bc<NP>(rv), V);
        g = (ev - t1) - t2;
        K.h[s][i] = h;
        K.rv[s][i] = rv;
#pragma unroll
        for (int c = 0; c < NC; ++c) L.xw[s][i][c] = W[c];
    }
    wave_prio<PRIO, 0>();
    __syncthreads();

    // O_k = S_{k,k+1} = -W_k' (transpose through LDS); S_{k,k-1} = -W_{k-1}
    float O[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float wt = L.xw[s][c][i < NC ? i : 0];
        O[c] = (i < NC) ? -wt : 0.0f;
        const float w = L.xw[sp][i][c];
        out.slo[c] = (has_prev && rowv) ? -w : 0.0f;
    }
    __syncthreads();

    // U_k = A_k Q~_k^-1 A_k' + B_k R_k^-1 B_k' = -(A_k O_k) + V_k B_k'
    {
        if constexpr (!SH::MMA) {
            float nar[NC], bcol[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                U[c] = 0.0f;
                nar[c] = -ar[c];
            }
            gemm_rows<NP, NC, NC>(U, BcRow<NP, NC>(O), nar);
            // lane i < m holds column i of B_k
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float bt = K.Bt[s][i < MC ? i : 0][c];
                bcol[c] = urow ? bt : 0.0f;
            }
            gemm_rows<NP, NC, MC>(U, BcRow<NP, NC>(bcol), V);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) L.xw[s][i][c] = U[c];
        L.xg[s][i] = g;
    }
    __syncthreads();

    // D_k = Q~_k^-1 + U_{k-1};  gamma_k = h + g_{k-1}  (gamma_0 = h + x0)
    float sd[NC];
    {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float qv = K.Q[s][i < NC ? i : 0][c];
            const float u = L.xw[sp][i][c];
            sd[c] = has_prev ? qv + u : qv;
        }
        const float gp = L.xg[sp][i];
        const float x0v = ld1(p.x0, (size_t)b * NC + i, rowv && k == 0);
        out.gam = rowv ? ((k >= 1) ? h + gp : h + x0v) : 0.0f;
    }
    __syncthreads();

    if constexpr (!PRE) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            out.sd[c] = rowv ? sd[c] : 0.0f;
            out.sup[c] = (rowv && k < N - 1) ? O[c] : 0.0f;
            out.plo[c] = out.pd[c] = out.pup[c] = 0.0f;
        }
        fl = 0;
        if (kv) {
            if (badq) fl |= GATO_F_Q_NOT_SPD;
            if (hn && badr) fl |= GATO_F_R_NOT_SPD;
        }
        return;
    }

    // D_k^-1
    wave_prio<PRIO, 3>();
    float di[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        di[c] = sd[c];
        out.sd[c] = rowv ? sd[c] : 0.0f;
    }
    inv_rows<SH, NC>(di, i, bads, L, s);
    wave_prio<PRIO, 0>();
    bads = group_any<SH::NP>(__builtin_amdgcn_ballot_w64(bads));
#pragma unroll
    for (int c = 0; c < NC; ++c) L.xw[s][i][c] = di[c];
    __syncthreads();

    // Phi^-1_{k,k+1} = -D_k^-1 O_k D_{k+1}^-1 ; Phi^-1_{k,k-1} = (Phi^-1_{k-1,k})'
    {
        const int sn = s + 1 < SL ? s + 1 : s;
        float Dn[NC], Y[NC], Z[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float d = L.xw[sn][i][c];
            Dn[c] = (s + 1 < SL) ? d : 0.0f;
            Y[c] = 0.0f;
            Z[c] = 0.0f;
        }
        __syncthreads();
        wave_prio<PRIO, 3>();
        if constexpr (SH::MMA) {
            // Z = D_k^-1 (O_k D_{k+1}^-1): Y holds the rows of (O_k D_{k+1}^-1)'
            mma_t<NP> acc = {};
            mma_abt<NC>(acc, Dn, O);
            mma_rows<NC>(acc, Y);
            acc = mma_t<NP>{};
            mma_abt<NC>(acc, di, Y);
            mma_rows<NC>(acc, Z);
        } else {
            gemm_rows<NP, NC, NC>(Y, BcRow<NP, NC>(O), di);  // Y = D_k^-1 O_k
            gemm_rows<NP, NC, NC>(Z, BcRow<NP, NC>(Dn), Y);  // Z = Y D_{k+1}^-1
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            L.xw[s][i][c] = Z[c];
            out.pup[c] = (rowv && k < N - 1) ? -Z[c] : 0.0f;
        }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float z = L.xw[sp][c][i < NC ? i : 0];
        out.plo[c] = (has_prev && rowv) ? -z : 0.0f;
        out.sup[c] = (rowv && k < N - 1) ? O[c] : 0.0f;
        out.pd[c] = rowv ? di[c] : 0.0f;
    }
    __syncthreads();
    wave_prio<PRIO, 0>();
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
    static constexpr bool kAssembled = true;  // applies the assembled Phi^-1 blocks
    static constexpr bool kPhased = false;    // Phi^-1 r in one call (see HybMat)
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
    __device__ __forceinline__ void sup(int, float (&out)[SH::NC]) const
    {
#pragma unroll
        for (int c = 0; c < SH::NC; ++c) out[c] = rw->sup[c];
    }
};

// Block-tridiagonal rows read from global memory at every product (for
// horizons longer than one workgroup holds); layout [B][N][3][n][n].
// Phi^-1 r in the stair preconditioner's factored form D^-1 (J S J) D^-1 r,
// D^-1 = blkdiag(Phi^-1_{k,k}) and J = blkdiag((-1)^k I), which equals the
// assembled blocks: y_j = D_j^-1 r_j for j = k-1, k, k+1, w_k = (J S J y)_k,
// then z_k = (D_k^-1)' w_k (column i).  r'z = y' J S J y then stays positive
// while S is SPD in fp32, even where the assembled fp32 Phi^-1 is not (its
// condition can exceed 1e8 on ill-conditioned long horizons, and the D_k^-1
// carry the rounding of their Gauss-Jordan inversion).
// PH (phased): y in two phases around one barrier, P1 forming y_k = D_k^-1 r_k
// (row i) and leaving it in the exchange rows xy, P2 taking the neighbours'
// y from there; D^-1 is then read twice per application instead of four
// times.  Without it (P) each lane forms y_{k-1} and y_{k+1} too, from the
// copies of r's neighbours the loop keeps; the bits are the same either way.
template <class SH, bool PH = true>
struct GlobalMat {
    static constexpr bool kAssembled = false;  // applies Phi^-1 in factored form
    static constexpr bool kPhased = PH;
    const float* Sm;
    const float* Pm;
    Ix<SH> ix;
    int b, i;
    float (*xy)[SH::NP];
    __device__ __forceinline__ float mv(const float* X, int k, float xp, float x, float xn) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        const bool v = k < ix.N && i < NC;
        float acc = 0.0f, t[NC];
        ld_row<NC>(X, ix.blk(b, k, 0, i), v, t);
        dotb<NP, NC>(acc, Bc<NP>(xp), t);
        ld_row<NC>(X, ix.blk(b, k, 1, i), v, t);
        dotb<NP, NC>(acc, Bc<NP>(x), t);
        ld_row<NC>(X, ix.blk(b, k, 2, i), v, t);
        dotb<NP, NC>(acc, Bc<NP>(xn), t);
        return acc;
    }
    __device__ __forceinline__ float S(int k, float xp, float x, float xn) const { return mv(Sm, k, xp, x, xn); }
    __device__ __forceinline__ float S(int k, float xp, float x, float xn, int) const { return mv(Sm, k, xp, x, xn); }
    __device__ __forceinline__ float P(int k, float rp, float r, float rn) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        const bool v = k < ix.N && i < NC;
        float t[NC], yp = 0.0f, y = 0.0f, yn = 0.0f, z = 0.0f;
        ld_row<NC>(Pm, ix.blk(b, k > 0 ? k - 1 : 0, 1, i), v && k > 0, t);
        dotb<NP, NC>(yp, Bc<NP>(rp), t);
        ld_row<NC>(Pm, ix.blk(b, k, 1, i), v, t);
        dotb<NP, NC>(y, Bc<NP>(r), t);
        ld_row<NC>(Pm, ix.blk(b, k + 1 < ix.N ? k + 1 : k, 1, i), v && k + 1 < ix.N, t);
        dotb<NP, NC>(yn, Bc<NP>(rn), t);
        const float w = mv(Sm, k, -yp, y, -yn);
        ld_row<NC, NC>(Pm, ix.blk(b, k, 1, 0) + i, v, t);  // column i of D_k^-1
        dotb<NP, NC>(z, Bc<NP>(w), t);
        return z;
    }
    __device__ __forceinline__ float P1(int k, float r) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        const bool v = k < ix.N && i < NC;
        float t[NC], y = 0.0f;
        ld_row<NC>(Pm, ix.blk(b, k, 1, i), v, t);
        dotb<NP, NC>(y, Bc<NP>(r), t);
        xy[k + 1][i] = y;
        return y;
    }
    __device__ __forceinline__ float P2(int k, float y, int) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        const bool v = k < ix.N && i < NC;
        const float w = mv(Sm, k, -xy[k][i], y, -xy[k + 2][i]);
        float t[NC], z = 0.0f;
        ld_row<NC, NC>(Pm, ix.blk(b, k, 1, 0) + i, v, t);  // column i of D_k^-1
        dotb<NP, NC>(z, Bc<NP>(w), t);
        return z;
    }
    __device__ __forceinline__ void sup(int k, float (&out)[SH::NC]) const
    {
        ld_row<SH::NC>(Sm, ix.blk(b, k, 2, i), k < ix.N && i < SH::NC, out);
    }
};

// The register-resident rows with Phi^-1 applied in its factored form
// D^-1 (J S J) D^-1, as GlobalMat applies it: y_k = D_k^-1 r_k (dsym: row i of
// D_k^-1 symmetrised) goes to the neighbouring groups through the exchange
// rows xy (one barrier), w_k = (J S J y)_k from the knot's S rows, z_k =
// D_k^-1 w_k.  With D_k^-1 symmetric, r'z = y' (J S J) y, positive while S is
// SPD in fp32.  One knot per lane group (C = 1).
template <class SH>
struct RegMatF : RegMat<SH> {
    static constexpr bool kAssembled = false;
    const float* dsym;
    float (*xy)[SH::NP];
    __device__ __forceinline__ float P(int k, float, float x, float) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        const int i = threadIdx.x % NP;
        float y = 0.0f, w = 0.0f, z = 0.0f;
        dotb<NP, NC>(y, Bc<NP>(x), dsym);
        xy[k + 1][i] = y;
        __syncthreads();
        const float yp = xy[k][i], yn = xy[k + 2][i];
        dotb<NP, NC>(w, Bc<NP>(-yp), this->rw->slo);
        dotb<NP, NC>(w, Bc<NP>(y), this->rw->sd);
        dotb<NP, NC>(w, Bc<NP>(-yn), this->rw->sup);
        dotb<NP, NC>(z, Bc<NP>(w), dsym);
        return z;
    }
};

// Rows for horizons of two knots per lane group (n <= 16), between RegMat and
// GlobalMat: S's diagonal blocks in registers (sd[c]: row i of S_{k,k} of the
// group's knot in chunk c), its off-diagonal blocks read from memory at every
// product, and the diagonal blocks D_k^-1 of the factored Phi^-1 in LDS
// (dinv[k][row][col]), read by rows for y = D^-1 r and by columns for
// z = D^-T w, in GlobalMat's two phases.  The products and their order are
// GlobalMat's, so the results are its bits, with the diagonal blocks read once
// instead of at every iteration.
template <class SH, int C, int DS>
struct HybMat {
    static constexpr bool kAssembled = false;
    static constexpr bool kPhased = true;
    const float* Sm;
    Ix<SH> ix;
    int b, i;
    const float (*sd)[SH::NC];
    const float (*dinv)[SH::NC][DS];
    float (*xy)[SH::NP];
    __device__ __forceinline__ float S(int k, float xp, float x, float xn, int c) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        const bool v = k < ix.N && i < NC;
        float acc = 0.0f, t[NC];
        ld_row<NC>(Sm, ix.blk(b, k, 0, i), v, t);
        dotb<NP, NC>(acc, Bc<NP>(xp), t);
        dotb<NP, NC>(acc, Bc<NP>(x), sd[c]);
        ld_row<NC>(Sm, ix.blk(b, k, 2, i), v, t);
        dotb<NP, NC>(acc, Bc<NP>(xn), t);
        return acc;
    }
    // y_k = D_k^-1 r_k (row i), left in the exchange rows for the neighbours
    __device__ __forceinline__ float P1(int k, float r) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        const bool v = k < ix.N && i < NC;
        float y = 0.0f;
        dotb<NP, NC>(y, Bc<NP>(r), dinv[k][v ? i : 0]);
        y = v ? y : 0.0f;
        xy[k + 1][i] = y;
        return y;
    }
    // after the barrier: w_k = (J S J y)_k, then z_k = (D_k^-1)' w_k (column i)
    __device__ __forceinline__ float P2(int k, float y, int c) const
    {
        constexpr int NP = SH::NP, NC = SH::NC;
        const bool v = k < ix.N && i < NC;
        const float w = S(k, -xy[k][i], y, -xy[k + 2][i], c);
        const int ii = i < NC ? i : 0;
        float col[NC], z = 0.0f;
#pragma unroll
        for (int r = 0; r < NC; ++r) col[r] = v ? dinv[k][r][ii] : 0.0f;
        dotb<NP, NC>(z, Bc<NP>(w), col);
        return z;
    }
    __device__ __forceinline__ void sup(int k, float (&out)[SH::NC]) const
    {
        ld_row<SH::NC>(Sm, ix.blk(b, k, 2, i), k < ix.N && i < SH::NC, out);
    }
};

// S p for the knot k of chunk c, for matrices that keep rows per chunk.
template <class MAT>
__device__ __forceinline__ float mat_S(const MAT& M, int c, int k, float xp, float x, float xn)
{
    if constexpr (MAT::kPhased) return M.S(k, xp, x, xn, c);
    else return M.S(k, xp, x, xn);
}

// Row i of (X + X')/2 for the row-per-lane block X of a lane group (lane i: row
// i in x), through the group's exchange row ex (NP floats, within one wave):
// column c of X is written there at step c and lane c reads it whole.
template <class SH>
__device__ __forceinline__ void sym_rows(const float* x, float* ex, float* out)
{
    constexpr int NC = SH::NC;
    const int i = threadIdx.x % SH::NP;
    float col[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) col[c] = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        ex[i] = x[c];
        __builtin_amdgcn_wave_barrier();
        if (i == c) {
#pragma unroll
            for (int c2 = 0; c2 < NC; ++c2) col[c2] = ex[c2];
        }
        __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) out[c] = 0.5f * (x[c] + col[c]);
}

// Leaves of the canonical knot sums: at least 64 and a power of two.
__host__ __device__ constexpr int leaves_for(int knots)
{
    int p = 64;
    while (p < knots) p *= 2;
    return p;
}

template <class SH, int C>
struct PcgLds {
    static constexpr int K = SH::SLOTS * C;  // knots held (C per lane group)
    static constexpr int P = leaves_for(K);  // canonical-sum leaves
    // exchange rows for knots -1 .. K (index + 1); rows 0 and K + 1 stay zero
    float xv[K + 2][SH::NP];
    float xz[K + 2][SH::NP];
    float xy[K + 2][SH::NP];    // y = D^-1 r of the factored Phi^-1 (RegMatF)
    alignas(16) float red0[P];  // per-knot partial sums: p'v
    alignas(16) float red1[P];  //                        r'r
    alignas(16) float red2[P];  //                        r'z
};

// Preconditioned CG on S lambda = gamma for one solve per workgroup (GATO
// paper Sec. II; the per-block PCG of Sec. III).  Each lane group owns C knots
// (k = c * SLOTS + s); per-knot partial sums go to LDS and every lane forms the
// same canonical total, so all waves take identical (scalar) branches.  Two
// workgroup barriers per iteration: after v = S p (for p'v and v's neighbours)
// and after z = Phi^-1 r (for r'r, r'z and z's neighbours).  Each lane keeps
// copies of the neighbouring knots' entries of r and p (same row), updated with
// the same arithmetic as their owners, so the products need no more exchange.
// lambda is accumulated in fp64: on ill-conditioned solves it sums hundreds of
// small steps, and in fp32 that sum alone would cost ~1e-3 in dz.
// Scheduling (the results are the same bits either way):
// - The step lengths alpha and beta are formed in vector registers from the
//   totals every lane holds (the same bits in each), so the updates do not wait
//   for a copy to scalar registers.
// - VS (vector stop), for one or two waves per SIMD: the stop test runs on the
//   vector unit too, with one scalar copy of its outcome for the loop's branch,
//   since there the test's scalar round trips sit on the iteration's critical
//   path.  With four waves per SIMD the vector unit is the busier one and the
//   test stays on the scalar unit; then (VS false) each phase between barriers
//   lowers the wave's priority as it goes (wave_prio: 3 for the chain after the
//   barrier, 2 for the product, 1 after it), and each wave stores its exchange
//   row before its partial sums, so that the store's latency, which the barrier
//   waits for, overlaps them.
// - RS: the residual's updates do not wait for the breakdown test (below).
// Internal stop code of pcg() (not a GATO_F_* bit): with the assembled Phi^-1,
// r'z <= 0 while the residual is above the tolerance, i.e. the fp32
// preconditioner is not positive definite on this solve.
constexpr int PCG_INDEFINITE = 1 << 16;

template <class SH, int C, class MAT, bool VS = false, bool RS = false>
__device__ __forceinline__ void pcg(const Params& p, const MAT& M, const float* gam, float* lam, PcgLds<SH, C>& L,
                                    int max_iters, int& iters_out, float& relres, int& flags_out)
{
    constexpr int NP = SH::NP, SL = SH::SLOTS, KK = PcgLds<SH, C>::K, P = PcgLds<SH, C>::P;
    constexpr int LPL = P / 16;  // leaves per lane of the canonical sum
    const int s = threadIdx.x / NP, i = threadIdx.x % NP;
    const bool lead = i == 0;
    const int nth = blockDim.x;

    // Zero what no lane group writes: the edge rows, the rows and leaves of
    // slots beyond the groups present (a block of G < SLOTS groups), and the
    // leaves past the last knot's.  Every other exchange row and leaf is
    // written by its own group before it is read, so these stores need no
    // barrier of their own.
    const int G = nth / NP;
    for (int t = threadIdx.x; t < P; t += nth)
        if (t >= KK || t % SL >= G) {
            L.red0[t] = 0.0f;
            L.red1[t] = 0.0f;
            L.red2[t] = 0.0f;
        }
    for (int t = threadIdx.x; t < (KK + 2) * NP; t += nth) {
        const int r = t / NP;
        if (r == 0 || r == KK + 1 || (r - 1) % SL >= G) {
            L.xv[r][t % NP] = 0.0f;
            L.xz[r][t % NP] = 0.0f;
            L.xy[r][t % NP] = 0.0f;
        }
    }

    auto row = [&](int c) { return c * SL + s + 1; };  // exchange row of chunk c

    // ||gamma||^2 and the neighbours of lambda
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const float t = groupsum<NP>(gam[c] * gam[c]);
        if (lead) L.red0[row(c) - 1] = t;
        L.xv[row(c)][i] = lam[c];
    }
    __syncthreads();
    const float gg = uniform(canon_sum<LPL>(L.red0));
    float lp[C], ln[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        lp[c] = L.xv[row(c) - 1][i];
        ln[c] = L.xv[row(c) + 1][i];
    }
    // (no barrier: xv is next written after the one that follows r's stores)

    int iters = 0, flags = 0;
    if (!__builtin_isfinite(gg)) {
        iters_out = 0;
        flags_out = GATO_F_NONFINITE;
        relres = __builtin_nanf("");
        return;
    }
    if (gg == 0.0f) {
#pragma unroll
        for (int c = 0; c < C; ++c) lam[c] = 0.0f;
        iters_out = 0;
        flags_out = 0;
        relres = 0.0f;
        return;
    }
    // ||r|| <= eps ||gamma||  <=>  r'r <= eps^2 gamma'gamma (both sides non-negative)
    const float tol2 = (p.eps * p.eps) * gg;

    // r = gamma - S lambda, and its neighbours
    float r[C], rp[C], rn[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        r[c] = gam[c] - mat_S(M, c, row(c) - 1, lp[c], lam[c], ln[c]);
        L.xz[row(c)][i] = r[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c) {
        rp[c] = L.xz[row(c) - 1][i];
        rn[c] = L.xz[row(c) + 1][i];
    }
    // (no barrier: z goes to xv and the red1/red2 leaves, which nobody reads
    // between the barriers around this point; xz is next written in the loop)

    double lamd[C];
#pragma unroll
    for (int c = 0; c < C; ++c) lamd[c] = (double)lam[c];

    // z = Phi^-1 r; r'r and r'z; neighbours of z
    float pv[C], pp[C], pn[C];
    float rr, eta;
    {
        float z[C];
        if constexpr (MAT::kPhased) {
            float y[C];
#pragma unroll
            for (int c = 0; c < C; ++c) y[c] = M.P1(row(c) - 1, r[c]);
            __syncthreads();
#pragma unroll
            for (int c = 0; c < C; ++c) z[c] = M.P2(row(c) - 1, y[c], c);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if constexpr (!MAT::kPhased) z[c] = M.P(row(c) - 1, rp[c], r[c], rn[c]);
            const float a = groupsum<NP>(r[c] * r[c]);
            const float bb = groupsum<NP>(r[c] * z[c]);
            if (lead) {
                L.red1[row(c) - 1] = a;
                L.red2[row(c) - 1] = bb;
            }
            L.xv[row(c)][i] = z[c];
        }
        __syncthreads();
        canon_sum2<LPL>(L.red1, L.red2, rr, eta);
        rr = uniform(rr);
        eta = uniform(eta);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            pp[c] = L.xv[row(c) - 1][i];
            pn[c] = L.xv[row(c) + 1][i];
            pv[c] = z[c];
        }
        __syncthreads();
    }
    if (!__builtin_isfinite(rr)) flags |= GATO_F_NONFINITE;
    if constexpr (MAT::kAssembled) {
        if (!(rr <= tol2) && !flags && !(eta > 0.0f)) flags |= PCG_INDEFINITE;
    }
    if (!(rr <= tol2) && !flags && iters >= max_iters) flags |= GATO_F_PCG_MAXITER;
    if (!(rr <= tol2) && !flags) {
        int itv = iters;
        // One exit, after the second barrier: a breakdown at the first one leaves
        // lambda, r and the count as they are and only sets the stop code, so every
        // loop-carried value has a single definition per iteration.
        for (;;) {
            // v = S p ; p'v ; v to neighbours
            wave_prio<!VS, 2>();
            float v[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                v[c] = mat_S(M, c, row(c) - 1, pp[c], pv[c], pn[c]);
                wave_prio<!VS, 1>();
                if constexpr (!VS) {
                    L.xv[row(c)][i] = v[c];  // first: the store overlaps the sum
                    mem_order();
                }
                const float t = groupsum<NP>(pv[c] * v[c]);
                if (lead) L.red0[row(c) - 1] = t;
                if constexpr (VS) L.xv[row(c)][i] = v[c];
            }
            __syncthreads();
            wave_prio<!VS, 3>();
            float vp[C], vn[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                vp[c] = L.xv[row(c) - 1][i];
                vn[c] = L.xv[row(c) + 1][i];
            }
            const float pSpv = canon_sum<LPL>(L.red0);
            const float pSp = VS ? pSpv : uniform(pSpv);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                pin(vp[c]);
                pin(vn[c]);
            }
            int stop1;
            if constexpr (VS)
                stop1 = !__builtin_isfinite(pSp) ? GATO_F_NONFINITE : !(pSp > 0.0f) ? GATO_F_PCG_BREAKDOWN : 0;
            else
                stop1 = !finite_bits(pSp) ? GATO_F_NONFINITE : !pos_bits(pSp) ? GATO_F_PCG_BREAKDOWN : 0;
            int stop = stop1;
            const float a = eta * __builtin_amdgcn_rcpf(pSpv);
            // A breakdown here ends the loop after the second barrier with lambda,
            // r and r'r as they were.  The updates select the old values; with RS
            // (for four waves per SIMD, where it pays) only lambda's does, r's are
            // made regardless, off the scalar stop test's path (r is not used after
            // the loop), and the old r'r is put back at the exit.
            const float rrk = rr;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const double l1 = fma((double)a, (double)pv[c], lamd[c]);
                const float r1 = fmaf(-a, v[c], r[c]);
                const float rp1 = fmaf(-a, vp[c], rp[c]);
                const float rn1 = fmaf(-a, vn[c], rn[c]);
                lamd[c] = stop ? lamd[c] : l1;
                if constexpr (!RS) {
                    r[c] = stop ? r[c] : r1;
                    rp[c] = stop ? rp[c] : rp1;
                    rn[c] = stop ? rn[c] : rn1;
                } else {
                    r[c] = r1;
                    rp[c] = rp1;
                    rn[c] = rn1;
                }
            }
            itv += stop ? 0 : 1;
            // z = Phi^-1 r ; r'r, r'z ; z to neighbours
            wave_prio<!VS, 2>();
            float z[C];
            if constexpr (MAT::kPhased) {
                float y[C];
#pragma unroll
                for (int c = 0; c < C; ++c) y[c] = M.P1(row(c) - 1, r[c]);
                __syncthreads();
#pragma unroll
                for (int c = 0; c < C; ++c) z[c] = M.P2(row(c) - 1, y[c], c);
            }
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if constexpr (!MAT::kPhased) z[c] = M.P(row(c) - 1, rp[c], r[c], rn[c]);
                wave_prio<!VS, 1>();
                if constexpr (!VS) {
                    L.xz[row(c)][i] = z[c];  // first: the store overlaps the sums
                    mem_order();
                }
                const float ta = groupsum<NP>(r[c] * r[c]);
                const float tb = groupsum<NP>(r[c] * z[c]);
                if (lead) {
                    L.red1[row(c) - 1] = ta;
                    L.red2[row(c) - 1] = tb;
                }
                if constexpr (VS) L.xz[row(c)][i] = z[c];
            }
            __syncthreads();
            wave_prio<!VS, 3>();
            float zp[C], zn[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                zp[c] = L.xz[row(c) - 1][i];
                zn[c] = L.xz[row(c) + 1][i];
            }
            float rrv, rzv;
            canon_sum2<LPL>(L.red1, L.red2, rrv, rzv);
            rr = VS ? rrv : uniform(rrv);
            const float rz = VS ? rzv : uniform(rzv);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                pin(zp[c]);
                pin(zn[c]);
            }
            // the first stop of the iteration holds; then, in this order of
            // precedence: r'r not finite, converged, r'z not finite, r'z <= 0
            // with the assembled Phi^-1, the cap (selects, one branch)
            {
                int st = itv >= max_iters ? GATO_F_PCG_MAXITER : 0;
                if constexpr (VS) {
                    st = (MAT::kAssembled && !(rz > 0.0f)) ? PCG_INDEFINITE : st;
                    st = !__builtin_isfinite(rz) ? GATO_F_NONFINITE : st;
                    st = rr <= tol2 ? -1 : st;  // converged
                    st = !__builtin_isfinite(rr) ? GATO_F_NONFINITE : st;
                } else {  // the same tests on the bits (rr >= 0 and tol2 > 0)
                    st = (MAT::kAssembled && !pos_bits(rz)) ? PCG_INDEFINITE : st;
                    st = !finite_bits(rz) ? GATO_F_NONFINITE : st;
                    st = le_nonneg_bits(rr, tol2) ? -1 : st;  // converged
                    st = !finite_bits(rr) ? GATO_F_NONFINITE : st;
                }
                stop = uniform_i(stop ? stop : st);
            }
            if (__builtin_expect(stop != 0, 0)) {
                flags |= stop > 0 ? stop : 0;
                if (RS && stop1) rr = rrk;
                break;
            }
            const float be = rzv * __builtin_amdgcn_rcpf(eta);
            eta = rz;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                pv[c] = fmaf(be, pv[c], z[c]);
                pp[c] = fmaf(be, pp[c], zp[c]);
                pn[c] = fmaf(be, pn[c], zn[c]);
            }
        }
        wave_prio<!VS, 0>();
        iters = uniform_i(itv);
        rr = uniform(rr);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) lam[c] = (float)lamd[c];
    iters_out = iters;
    flags_out = flags;
    relres = sqrtf(rr / gg);
    // The loop's barriers order every LDS access above; one more before the
    // caller reuses the buffers.
    __syncthreads();
}

// PCG as above within p.max_iters iterations in all.  With the assembled Phi^-1
// a solve whose r'z stops being positive (its fp32 blocks can be indefinite
// where cond(Phi^-1) passes ~1e8) switches at that iteration to Phi^-1 in
// factored form and restarts from its current lambda with the iterations left;
// iters counts both runs.  The decision is uniform over the workgroup (one
// solve), and a solve whose r'z stays positive never takes it.
template <class SH, int C, class MAT, bool VS = false, bool RS = false>
__device__ __forceinline__ void pcg_robust(const Params& p, const MAT& M, const float* gam, float* lam,
                                           PcgLds<SH, C>& L, int& iters_out, float& relres, int& flags_out)
{
    pcg<SH, C, MAT, VS, RS>(p, M, gam, lam, L, p.max_iters, iters_out, relres, flags_out);
    if constexpr (MAT::kAssembled) {
        static_assert(C == 1, "one knot per lane group");
        if (flags_out == PCG_INDEFINITE) {
            const int left = p.max_iters - iters_out;
            if (left <= 0) {
                flags_out = GATO_F_PCG_MAXITER;
            } else {
                float dsym[SH::NC];
                sym_rows<SH>(M.rw->pd, L.xy[threadIdx.x / SH::NP + 1], dsym);
                const RegMatF<SH> F{{M.rw}, dsym, L.xy};
                int it2 = 0, fl2 = 0;
                pcg<SH, C, RegMatF<SH>, VS, RS>(p, F, gam, lam, L, left, it2, relres, fl2);
                iters_out += it2;
                flags_out = fl2;
            }
        }
    }
}

// ------------------------------------------------------------------ stage 2b: recovery

// dx_k = Q~_k^-1 (lambda_k - A_k' lambda_{k+1} - q_k), du_k = R_k^-1 (-B_k' lambda_{k+1} - r_k)
// (the back-substitution of the Schur solve, GATO paper Sec. II eq. 4).  The
// A_k term is taken from the upper block of S, S_{k,k+1} = -Q~_k^-1 A_k', so
//   dx_k = Q~_k^-1 lambda_k + S_{k,k+1} lambda_{k+1} - Q~_k^-1 q_k,
// which needs no A_k.  Lane i holds row i of Q~_k^-1, S_{k,k+1} and R_k^-1,
// column i of B_k, (Q~_k^-1 q_k)_i as h and (r_k)_i as rv.
template <class SH>
__device__ __forceinline__ void recover(int i, bool rowv, bool urow, float lam, float lamn, const float* qi,
                                        const float* sup, float h, const float* bcol, float rv, const float* ri,
                                        float& dx, float& du)
{
    constexpr int NC = SH::NC, MC = SH::MC, NP = SH::NP;
    const Bc<NP> lnb(lamn);
    float x = 0.0f, tb = 0.0f;
    dotb<NP, NC>(x, Bc<NP>(lam), qi);
    dotb<NP, NC>(x, lnb, sup);
    dotb<NP, NC>(tb, lnb, bcol);
    const float u = urow ? -tb - rv : 0.0f;
    float y = 0.0f;
    dotb<NP, MC>(y, Bc<NP>(u), ri);
    dx = rowv ? x - h : 0.0f;
    du = urow ? y : 0.0f;
}

// ------------------------------------------------------------------ refinement residual

// Lane i's rows of the residual of the KKT system the Schur method solves
// (G dz - C' lambda = -g, C dz = c; GATO paper Sec. II, eq. 2) at knot k, the
// right-hand side of one pass of iterative refinement:
//   q'_k = q_k + Q~_k dx_k - lambda_k + A_k' lambda_{k+1}
//   r'_k = r_k + R_k du_k + B_k' lambda_{k+1}
//   e'_k = e_k + A_k dx_k + B_k du_k - dx_{k+1}
//   x0'  = x0 - dx_0                                     (k = 0)
// accumulated in double from the fp32 problem data and rounded once.  dx, du,
// ln: dx_k, du_k and lambda_{k+1} whole (any memory every lane can read);
// lam: (lambda_k)_i; dxn: (dx_{k+1})_i.  Rows and knots outside the problem
// give zeros.  SEQ: one row of the problem data in registers at a time (each
// product is summed before the next row is requested), for callers that keep
// many registers live across this.
template <class SH, bool SEQ = false>
__device__ __forceinline__ void kkt_rows(const Params& p, int b, int k, int i, bool kv, const float* dx,
                                         const float* du, const float* ln, float lam, float dxn, float& qv,
                                         float& rv, float& ev, float& x0v)
{
    auto step = [](double x) {
        if constexpr (SEQ) seq_after(x);
    };
    constexpr int n = SH::NC, m = SH::MC;
    const Ix<SH> ix{p.N};
    const bool dyn = kv && k < p.N - 1;
    qv = rv = ev = x0v = 0.0f;
    if (kv && i < n) {
        const double rh = p.rho != nullptr ? (double)p.rho[b] : 0.0;
        double s = (double)p.q[ix.vn(b, k, i)] + rh * dx[i] - lam;
        const float* Qr = p.Q + ix.Q(b, k, i);
#pragma unroll
        for (int c = 0; c < n; ++c) s += (double)Qr[c] * dx[c];
        step(s);
        if (dyn) {
            const float* Ac = p.A + ix.A(b, k, 0) + i;  // column i of A_k
#pragma unroll
            for (int c = 0; c < n; ++c) s += (double)Ac[c * n] * ln[c];
            step(s);
            const float* Ar = p.A + ix.A(b, k, i);
            const float* Br = p.Bu + ix.Bu(b, k, i);
            double t = (double)p.e[ix.e(b, k, i)] - dxn;
#pragma unroll
            for (int c = 0; c < n; ++c) t += (double)Ar[c] * dx[c];
            step(t);
#pragma unroll
            for (int c = 0; c < m; ++c) t += (double)Br[c] * du[c];
            step(t);
            ev = (float)t;
        }
        qv = (float)s;
        if (k == 0) x0v = (float)((double)p.x0[(size_t)b * n + i] - dx[i]);
    }
    if (dyn && i < m) {
        double s = (double)p.r[ix.vm(b, k, i)];
        const float* Rr = p.R + ix.R(b, k, i);
#pragma unroll
        for (int c = 0; c < m; ++c) s += (double)Rr[c] * du[c];
        step(s);
        const float* Bc_ = p.Bu + ix.Bu(b, k, 0) + i;  // column i of B_k
#pragma unroll
        for (int c = 0; c < n; ++c) s += (double)Bc_[c * m] * ln[c];
        rv = (float)s;
    }
}

// ------------------------------------------------------------------ stage 2, direct

// Direct solve of S lambda = gamma for block-tridiagonal SPD S by block
// elimination (block Thomas, the block LDL' factorisation of S), then the
// recovery of dz.  This is the alternative to PCG that the GATO pages discuss
// for long horizons (the paper's block-tridiagonal direct solve; Branch's
// chronological elimination of block-structured KKT systems).
//   H_0 = D_0,  g_0 = gamma_0;
//   T_k = S_{k,k-1} H_{k-1}^-1,  H_k = D_k - T_k S_{k-1,k},  g_k = gamma_k - T_k g_{k-1};
//   lambda_{N-1} = H_{N-1}^-1 g_{N-1},  lambda_k = H_k^-1 (g_k - S_{k,k+1} lambda_{k+1}).
// Every H_k is SPD when S is (a Schur complement of a leading block of S), so
// the Gauss-Jordan inversion runs without pivoting; a pivot that is not
// positive sets S_NOT_SPD.  One lane group holds one solve and walks the knots
// in order (lane i: row i of every block); H_k^-1 rows and g_k go to the
// workspace on the way down and are read back on the way up, where each
// knot's dz is recovered as soon as lambda_k is known.  The next knot's rows
// are requested before the current knot's arithmetic.
template <class SH>
__device__ __forceinline__ void direct_solve(const Params& p, int b, bool bv, float* pr)
{
    constexpr int NP = SH::NP, NC = SH::NC, MC = SH::MC;
    const Ix<SH> ix{p.N};
    const int N = p.N;
    const int i = threadIdx.x % NP;
    const int bb = bv ? b : 0;  // lane groups without a solve read masked rows of solve 0
    const bool rowi = bv && i < NC;
    float* Hw = p.dws;
    float* Gw = p.dws + (size_t)p.B * N * NC * NC;
    const size_t hrow = ((size_t)bb * N * NC + i) * NC;  // + k * NC * NC: row i of H_k^-1
    const size_t grow = (size_t)bb * N * NC + i;         // + k * NC

    // forward elimination
    bool bad = false;
    float Hi[NC], Sp[NC], gh = 0.0f;  // row i of H_{k-1}^-1 and S_{k-1,k}; g_{k-1} entry
    float lo[NC], dd[NC], up[NC], gam;
    ld_row<NC>(p.S, ix.blk(bb, 0, 0, i), rowi, lo);
    ld_row<NC>(p.S, ix.blk(bb, 0, 1, i), rowi, dd);
    ld_row<NC>(p.S, ix.blk(bb, 0, 2, i), rowi, up);
    gam = ld1(p.gamma, ix.vn(bb, 0, i), rowi);
#pragma unroll
    for (int c = 0; c < NC; ++c) Hi[c] = Sp[c] = 0.0f;
    for (int k = 0; k < N; ++k) {
        const bool nv = rowi && k + 1 < N;
        const int kn = k + 1 < N ? k + 1 : k;
        float nlo[NC], nd[NC], nup[NC];
        ld_row<NC>(p.S, ix.blk(bb, kn, 0, i), nv, nlo);
        ld_row<NC>(p.S, ix.blk(bb, kn, 1, i), nv, nd);
        ld_row<NC>(p.S, ix.blk(bb, kn, 2, i), nv, nup);
        const float ngam = ld1(p.gamma, ix.vn(bb, kn, i), nv);

        float T[NC], U[NC], H[NC];
        if constexpr (SH::MMA) {
            // on the matrix cores, with S_{k-1,k} = S_{k,k-1}' (S is symmetric)
            mma_t<NP> acc = {};
            mma_abt<NC>(acc, lo, Hi);  // T = S_{k,k-1} H_{k-1}^-1' (H_{k-1}^-1 symmetric; zero at k = 0)
            mma_rows<NC>(acc, T);
            acc = mma_t<NP>{};
            mma_abt<NC>(acc, T, lo);  // U = T S_{k,k-1}'
            mma_rows<NC>(acc, U);
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) T[c] = U[c] = 0.0f;
            gemm_rows<NP, NC, NC>(T, BcRow<NP, NC>(Hi), lo);  // T = S_{k,k-1} H_{k-1}^-1 (zero at k = 0)
            gemm_rows<NP, NC, NC>(U, BcRow<NP, NC>(Sp), T);   // U = T S_{k-1,k}
        }
        float tg = 0.0f;
        dotb<NP, NC>(tg, Bc<NP>(gh), T);
        const float gk = gam - tg;
#pragma unroll
        for (int c = 0; c < NC; ++c) H[c] = (c == i && !rowi) ? 1.0f : dd[c] - U[c];  // identity rows off the problem
        bool bk = false;
        if constexpr (NP == 32) gj_steps_lds<NC>(H, i, bk, pr);
        else gj_steps<NP, NC>(H, i, bk);
        bad |= bk;
        if (rowi) {
#pragma unroll
            for (int c = 0; c < NC; ++c) Hw[hrow + (size_t)k * NC * NC + c] = H[c];
            Gw[grow + (size_t)k * NC] = gk;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            Hi[c] = H[c];
            Sp[c] = up[c];
            lo[c] = nlo[c];
            dd[c] = nd[c];
            up[c] = nup[c];
        }
        gh = gk;
        gam = ngam;
    }

    // back substitution, with the recovery of each knot's dz; the next knot's
    // rows are requested before this knot's arithmetic
    struct Back {
        float Hk[NC], sup[NC], qi[NC], ri[MC], bc[NC], gk, qv, rv;
    };
    auto fetch = [&](int k, Back& f) {
        const bool kok = rowi && k >= 0;
        const int kk = k >= 0 ? k : 0;
        const bool urow = kok && kk < N - 1 && i < MC;
        ld_row<NC>(Hw, hrow + (size_t)kk * NC * NC, kok, f.Hk);
        f.gk = ld1(Gw, grow + (size_t)kk * NC, kok);
        ld_row<NC>(p.S, ix.blk(bb, kk, 2, i), kok, f.sup);
        ld_row<NC>(p.Qinv, ix.Q(bb, kk, i), kok, f.qi);
        ld_row<MC>(p.Rinv, ix.R(bb, kk, i), urow, f.ri);
        ld_row<NC, MC>(p.Bu, ix.Bu(bb, kk, 0) + i, urow, f.bc);  // column i of B_k
        f.qv = ld1(p.q, ix.vn(bb, kk, i), kok);
        f.rv = ld1(p.r, ix.vm(bb, kk, i), urow);
    };
    bool nonfinite = false;
    float lamn = 0.0f;  // row i of lambda_{k+1}
    Back cur;
    fetch(N - 1, cur);
    for (int k = N - 1; k >= 0; --k) {
        Back nxt;
        fetch(k - 1, nxt);
        const bool hn = bv && k < N - 1;
        const bool rowv = rowi;
        const bool urow = hn && i < MC;
        const float* Hk = cur.Hk;
        const float* sup = cur.sup;
        const float* qi = cur.qi;
        const float* ri = cur.ri;
        const float* bc = cur.bc;
        const float gk = cur.gk, qv = cur.qv, rv = cur.rv;

        float t = 0.0f;
        dotb<NP, NC>(t, Bc<NP>(lamn), sup);
        t = gk - t;  // g_k - S_{k,k+1} lambda_{k+1}
        float lam = 0.0f;
        dotb<NP, NC>(lam, Bc<NP>(t), Hk);
        lam = rowi ? lam : 0.0f;
        nonfinite |= rowi && !__builtin_isfinite(lam);
        float h = 0.0f;  // (Q~_k^-1 q_k)_i, as the formation forms it
        dotb<NP, NC>(h, Bc<NP>(qv), qi);
        float dx, du;
        recover<SH>(i, rowv, urow, lam, lamn, qi, sup, h, bc, rv, ri, dx, du);
        if (rowv) {
            p.lambda[ix.vn(bb, k, i)] = lam;
            p.dz[ix.dx(bb, k, i)] = dx;
        }
        if (urow) p.dz[ix.du(bb, k, i)] = du;
        lamn = lam;
        cur = nxt;
    }

    // per-solve flags: any lane of the group
    const uint64_t grp = (NP == 64 ? ~0ull : ((1ull << NP) - 1ull)) << (threadIdx.x & (64 - NP));
    const bool any_bad = (__builtin_amdgcn_ballot_w64(bad && rowi) & grp) != 0;
    const bool any_nf = (__builtin_amdgcn_ballot_w64(nonfinite) & grp) != 0;
    if (bv && i == 0) {
        int fl = p.flags[b];
        if (any_bad) fl |= GATO_F_S_NOT_SPD;
        if (any_nf) fl |= GATO_F_NONFINITE;
        p.flags[b] = fl;
        if (p.iters) p.iters[b] = 0;
        if (p.relres) p.relres[b] = 0.0f;
    }
}

// ------------------------------------------------------------------ stage 3: merit

// The problem rows and entries one lane needs for its knot's merit terms:
// row i of Q_k, A_k (n wide), R_k and B_k (m wide), and q, r, e, x0 entries;
// zeros where the row or entry does not exist.
template <class SH>
struct MeritIn {
    float Q[SH::NC], A[SH::NC], R[SH::MC], B[SH::MC];
    float q, r, e, x0;
};

template <class SH>
__device__ __forceinline__ void merit_rows(const Params& p, int b, int k, int i, MeritIn<SH>& in)
{
    constexpr int NC = SH::NC, MC = SH::MC;
    const Ix<SH> ix{p.N};
    const bool kv = k < p.N, hn = kv && k < p.N - 1, rowv = kv && i < NC, urow = hn && i < MC;
    ld_row<NC>(p.Q, ix.Q(b, k, i), rowv, in.Q);
    ld_row<NC>(p.A, ix.A(b, k, i), hn && i < NC, in.A);
    ld_row<MC>(p.R, ix.R(b, k, i), urow, in.R);
    ld_row<MC>(p.Bu, ix.Bu(b, k, i), hn && i < NC, in.B);
    in.q = ld1(p.q, ix.vn(b, k, i), rowv);
    in.r = ld1(p.r, ix.vm(b, k, i), urow);
    in.e = ld1(p.e, ix.e(b, k, i), hn && i < NC);
    in.x0 = ld1(p.x0, (size_t)b * NC + i, rowv && k == 0);
}

// Per-knot merit terms at a = 0 and at every step size (GATO paper Sec. II
// eq. 3; Sec. III eq. 7):
//   m_k(a) = a LIN + (a^2/2) QUAD + mu L1(a),
//   LIN = q'dx + r'du,  QUAD = dx'Q dx + du'R du  (undamped Q),
//   L1(a) = ||e_k + a (A dx + B du - dx_{k+1})||_1 + [k = 0] ||x0 - a dx_0||_1.
// Sums over the lanes of a group use the canonical butterfly and every rounding
// is explicit, so a knot's values do not depend on the kernel computing them.
//
// The step-size-independent part of a knot's merit terms: LIN, QUAD (summed
// over the knot's lanes) and this lane's entry of A dx + B du - dx_{k+1}.
struct MeritPrep {
    float lin, quad, d;
};

template <class SH>
__device__ __forceinline__ MeritPrep merit_prep(const Params& p, int k, const MeritIn<SH>& in, float dx, float du,
                                                float dxn)
{
    constexpr int NC = SH::NC, MC = SH::MC, NP = SH::NP;
    const bool hn = k < p.N - 1;
    const Bc<NP> xb(dx), ub(du);
    float Qdx = 0.0f, Rdu = 0.0f, d = 0.0f;
    dotb<NP, NC>(Qdx, xb, in.Q);
    dotb<NP, MC>(Rdu, ub, in.R);
    dotb<NP, NC>(d, xb, in.A);
    dotb<NP, MC>(d, ub, in.B);
    MeritPrep m;
    m.d = hn ? __fsub_rn(d, dxn) : 0.0f;
    m.lin = groupsum<NP>(__fadd_rn(__fmul_rn(in.q, dx), __fmul_rn(in.r, du)));
    m.quad = groupsum<NP>(__fadd_rn(__fmul_rn(dx, Qdx), __fmul_rn(du, Rdu)));
    return m;
}

// A knot's merit term at step size j (j = 0: a = 0), in every lane of the group.
template <class SH>
__device__ __forceinline__ float merit_value(const Params& p, int k, const MeritIn<SH>& in, const MeritPrep& m,
                                             float dx, int j)
{
    const float a = (j == 0) ? 0.0f : p.alphas[j - 1];
    float l1 = fabsf(__fmaf_rn(a, m.d, in.e));
    const float l0 = __fadd_rn(l1, fabsf(__fmaf_rn(-a, dx, in.x0)));
    l1 = (k == 0) ? l0 : l1;
    const float L1 = groupsum<SH::NP>(l1);
    return __fadd_rn(__fadd_rn(__fmul_rn(a, m.lin), __fmul_rn(__fmul_rn(0.5f, __fmul_rn(a, a)), m.quad)),
                     __fmul_rn(p.mu, L1));
}

// All step sizes of one knot: the group's lane 0 writes value j (j = 0: a = 0)
// to out[j * stride].
template <class SH>
__device__ __forceinline__ void merit_knot(const Params& p, int k, int i, const MeritIn<SH>& in, float dx, float du,
                                           float dxn, float* out, int stride)
{
    const bool kv = k < p.N;
    const MeritPrep m = merit_prep<SH>(p, k, in, dx, du, dxn);
#pragma unroll 1
    for (int j = 0; j <= GATO_MAX_ALPHA; ++j) {
        if (j <= p.n_alpha) {
            const float val = merit_value<SH>(p, k, in, m, dx, j);
            if (i == 0 && kv) out[j * stride] = val;
        }
    }
}

// Canonical sums of the per-knot merit values and the step selection
// (argmin, ties to the earlier step; accepted only below merit0).  Only wave 0
// takes part: its four 16-lane rows form the sums of different step sizes side
// by side (row r takes j = r, r + 4, ...), row leaders store them, and every
// lane of the wave reads them back in j order for the selection.  Returns
// false in the other waves (best and lsfail are then not set).
template <int LPL>
__device__ __forceinline__ bool merit_select(const Params& p, int b, const float* vals, int P, int32_t& best,
                                             int& lsfail)
{
    constexpr int RMAX = (GATO_MAX_ALPHA + 1 + 3) / 4;
    if (threadIdx.x >= 64) return false;
    const int r = threadIdx.x >> 4;
    const int na = p.n_alpha;
    float sum[RMAX];
#pragma unroll
    for (int q = 0; q < RMAX; ++q) {
        if (4 * q <= na) {
            const int j = 4 * q + r;
            sum[q] = canon_sum<LPL>(vals + (j <= na ? j : na) * P);
            if ((threadIdx.x & 15) == 0 && j >= 1 && j <= na) p.merit[(size_t)b * na + (j - 1)] = sum[q];
        }
    }
    const float M0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum[0]), 0));
    if (threadIdx.x == 0) p.merit0[b] = M0;
    float bv = 0.0f;
    int bi = 0;
#pragma unroll
    for (int j = 1; j <= GATO_MAX_ALPHA; ++j) {
        if (j <= na) {
            const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum[j / 4]), 16 * (j % 4)));
            if (j == 1 || v < bv) {
                bv = v;
                bi = j - 1;
            }
        }
    }
    lsfail = !(bv < M0);
    best = lsfail ? -1 : bi;
    return true;
}

}  // namespace gato
