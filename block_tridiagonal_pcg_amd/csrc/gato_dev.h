// gato_dev.h -- lane-level building blocks for the gfx950 kernels.
//
// Data layout inside a workgroup: every knot point owns one group of NP lanes
// (NP = 16 for n <= 16, NP = 32 for n <= 32); lane i of the group holds row i
// of that knot's blocks in registers.  A wave64 therefore holds 64/NP knots.
// Products of the small per-knot blocks broadcast a value of lane l of the
// group to the whole group with the DPP `row_newbcast` control, folded into the
// multiply-add (see dpp_asm.inc), so the block-dense linear algebra of one knot
// needs no LDS traffic.  For NP = 32 a group spans two DPP rows; a broadcast
// then reads from a copy in which V_PERMLANE16_SWAP has duplicated the lower
// (or upper) row of the group into both rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gato {

#include "dpp_asm.inc"

// Compile-time shape of one instantiation.
//   NC, MC: loop bounds for states and controls (runtime n <= NC, m <= MC;
//           rows/columns beyond n, m are zero and padded diagonals are one).
//   NP:     lanes per knot; SLOTS: knots one workgroup holds (by default the
//           most a 1024-thread workgroup holds; fewer for the windowed formation).
template <int NC_, int MC_, int SLOTS_ = 0>
struct Shape {
    static constexpr int NC = NC_;
    static constexpr int MC = MC_;
    static constexpr int NP = NC_ <= 16 ? 16 : 32;
    static constexpr int KPW = 64 / NP;
    static constexpr int SLOTS = SLOTS_ ? SLOTS_ : (NP == 16 ? 64 : 16);
    static constexpr int THREADS = SLOTS * NP;
    // Whether the formation's n x n products go to the matrix cores: a
    // 16x16x1 MFMA step costs as much as ~7 DPP multiply-adds per row, a
    // 32x32x1 step as much as ~15 (and 32-lane broadcasts also pay a permlane).
    static constexpr bool MMA = (NP == 16 && NC_ >= 8) || (NP == 32 && NC_ >= 16);
    static_assert(MC_ <= NC_ || MC_ <= NP, "controls must fit in a knot's lane group");
};

// ------------------------------------------------------------------ DPP moves

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double x)
{
    const int lo = __double2loint(x), hi = __double2hiint(x);
    const int l2 = __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xF, 0xF, false);
    const int h2 = __builtin_amdgcn_update_dpp(0, hi, CTRL, 0xF, 0xF, false);
    return __hiloint2double(h2, l2);
}

template <int CTRL, typename T>
__device__ __forceinline__ T dpp(T x)
{
    if constexpr (sizeof(T) == 8) return dpp_d<CTRL>(x);
    else return dpp_f<CTRL>(x);
}

constexpr int DPP_QP_1032 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QP_2301 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;

// Duplicate the even (lo) and odd (hi) 16-lane rows of every 32-lane pair.
__device__ __forceinline__ void dup_rows(float x, float& lo, float& hi)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}

__device__ __forceinline__ double pair_other(double x, bool upper)
{
    // value of the same lane in the other row of the 32-lane pair
    float lo0, hi0, lo1, hi1;
    dup_rows(__int_as_float(__double2loint(x)), lo0, hi0);
    dup_rows(__int_as_float(__double2hiint(x)), lo1, hi1);
    const float l = upper ? lo0 : hi0, h = upper ? lo1 : hi1;
    return __hiloint2double(__float_as_int(h), __float_as_int(l));
}

// Sum over the 16 lanes of each DPP row as the canonical pairwise tree
// ((x0+x1)+(x2+x3)) + ... ; every lane of the row ends with identical bits
// (each step adds a lane's value to its partner's, and IEEE addition commutes).
template <typename T>
__device__ __forceinline__ T rowsum16(T x)
{
    x = x + dpp<DPP_QP_1032>(x);
    x = x + dpp<DPP_QP_2301>(x);
    x = x + dpp<DPP_ROW_HALF_MIRROR>(x);
    x = x + dpp<DPP_ROW_MIRROR>(x);
    return x;
}

// Sum over the NP lanes of a knot group (canonical tree over NP leaves).
template <int NP, typename T>
__device__ __forceinline__ T groupsum(T x)
{
    x = rowsum16(x);
    if constexpr (NP == 32) {
        if constexpr (sizeof(T) == 8) {
            const bool upper = (threadIdx.x & 16) != 0;
            const T o = pair_other(x, upper);
            x = upper ? o + x : x + o;  // lower row's sum first, in both rows
        } else {
            float lo, hi;
            dup_rows(x, lo, hi);
            x = lo + hi;
        }
    }
    return x;
}

// Canonical pairwise sum of P = 16 * L leaves held in LDS (zero-padded, 16-byte
// aligned, L a multiple of 4), in every lane: lane j of each 16-lane row reads
// leaves [j L, (j+1) L) with 16-byte loads and sums them pairwise, and the row
// butterfly combines the 16 partial sums.  Every node of the tree adds two
// equal-sized contiguous halves, so the result is the pairwise tree over the P
// leaves whatever kernel or block shape computes it, and with zero padding it
// equals the tree over the smallest power of two >= the number of real leaves.
template <int L>
__device__ __forceinline__ void canon_leaves(const float* leaves, float (&v)[L])
{
    static_assert(L % 4 == 0, "leaves are read four at a time");
    const float4* q = reinterpret_cast<const float4*>(leaves) + (threadIdx.x & 15) * (L / 4);
#pragma unroll
    for (int t = 0; t < L / 4; ++t) {
        const float4 f = q[t];
        v[4 * t] = f.x;
        v[4 * t + 1] = f.y;
        v[4 * t + 2] = f.z;
        v[4 * t + 3] = f.w;
    }
}

template <int L>
__device__ __forceinline__ float canon_tree(float (&v)[L])
{
#pragma unroll
    for (int w = 1; w < L; w *= 2)
#pragma unroll
        for (int t = 0; t < L; t += 2 * w) v[t] = v[t] + v[t + w];
    return rowsum16(v[0]);
}

template <int L>
__device__ __forceinline__ float canon_sum(const float* leaves)
{
    float v[L];
    canon_leaves<L>(leaves, v);
    return canon_tree<L>(v);
}

// Two canonical sums with their loads issued together.
template <int L>
__device__ __forceinline__ void canon_sum2(const float* la, const float* lb, float& a, float& b)
{
    float va[L], vb[L];
    canon_leaves<L>(la, va);
    canon_leaves<L>(lb, vb);
#pragma unroll
    for (int w = 1; w < L; w *= 2)
#pragma unroll
        for (int t = 0; t < L; t += 2 * w) {
            va[t] = va[t] + va[t + w];
            vb[t] = vb[t] + vb[t + w];
        }
    a = va[0] + dpp<DPP_QP_1032>(va[0]);
    b = vb[0] + dpp<DPP_QP_1032>(vb[0]);
    a = a + dpp<DPP_QP_2301>(a);
    b = b + dpp<DPP_QP_2301>(b);
    a = a + dpp<DPP_ROW_HALF_MIRROR>(a);
    b = b + dpp<DPP_ROW_HALF_MIRROR>(b);
    a = a + dpp<DPP_ROW_MIRROR>(a);
    b = b + dpp<DPP_ROW_MIRROR>(b);
}

// ------------------------------------------------------------------ broadcast sources

// A value to be broadcast from any lane of a knot group.
template <int NP>
struct Bc;
template <>
struct Bc<16> {
    float lo;
    __device__ __forceinline__ explicit Bc(float x) : lo(x) {}
};
template <>
struct Bc<32> {
    float lo, hi;
    __device__ __forceinline__ explicit Bc(float x) { dup_rows(x, lo, hi); }
};

// acc += sum_{c < K} x(lane c) * row[c]
template <int NP, int K>
__device__ __forceinline__ void dotb(float& acc, const Bc<NP>& x, const float* row)
{
    if constexpr (NP == 16) {
        static_assert(K <= 16, "");
        bcA<K>(acc, x.lo, row);
    } else {
        static_assert(K <= 32, "");
        bcA<(K < 16 ? K : 16)>(acc, x.lo, row);
        if constexpr (K > 16) bcA<K - 16>(acc, x.hi, row + 16);
    }
}

// Row arrays to be broadcast from a fixed lane (one register per column).
template <int NP, int K>
struct BcRow;
template <int K>
struct BcRow<16, K> {
    float lo[K];
    __device__ __forceinline__ explicit BcRow(const float* x)
    {
#pragma unroll
        for (int c = 0; c < K; ++c) lo[c] = x[c];
    }
};
template <int K>
struct BcRow<32, K> {
    float lo[K], hi[K];
    __device__ __forceinline__ explicit BcRow(const float* x)
    {
#pragma unroll
        for (int c = 0; c < K; ++c) dup_rows(x[c], lo[c], hi[c]);
    }
};

template <int K, int L>
__device__ __forceinline__ void bcB_chunks(float* acc, const float* src, float mul)
{
    if constexpr (K <= 16) {
        BcB<K>::template run<L>(acc, src, mul);
    } else {
        BcB<16>::template run<L>(acc, src, mul);
        bcB_chunks<K - 16, L>(acc + 16, src + 16, mul);
    }
}

// acc[c] += x[c](lane L) * mul for c < K
template <int NP, int K, int L>
__device__ __forceinline__ void axpyb(float* acc, const BcRow<NP, K>& x, float mul)
{
    if constexpr (NP == 16) {
        bcB_chunks<K, L>(acc, x.lo, mul);
    } else {
        if constexpr (L < 16) bcB_chunks<K, L>(acc, x.lo, mul);
        else bcB_chunks<K, L - 16>(acc, x.hi, mul);
    }
}

// acc[c] += sum_{l < KL} X[l][c] * mul[l], X's row l held by lane l (outer products).
template <int NP, int K, int KL, int L = 0>
__device__ __forceinline__ void gemm_rows(float* acc, const BcRow<NP, K>& x, const float* mul)
{
    if constexpr (L < KL) {
        axpyb<NP, K, L>(acc, x, mul[L]);
        gemm_rows<NP, K, KL, L + 1>(acc, x, mul);
    }
}

// ------------------------------------------------------------------ matrix-core products

// A product A B' of a wave's knots at once on the matrix cores, with A, B and
// the result all in row layout (lane i of a group holds row i).  One MFMA step
// per k: V_MFMA_F32_16X16X1_4B_F32 for 16-lane groups (four 16x16 blocks, one
// per group), V_MFMA_F32_32X32X1_2B_F32 for 32-lane groups (two 32x32 blocks).
// Lane i of a group supplies B[i][k] as the first operand and A[i][k] as the
// second, so each block accumulates D = B A'.
//   16 lanes: D[a][b] sits in lane 16*(a/4) + b, register 4*group + a%4.
//             `mma_rows` moves tile (lane row q, register quartet g) to (lane
//             row g, quartet q) with two rounds of permlane swaps.
//   32 lanes: D[a][b] sits in lane 32*((a/4)%2) + b, register
//             16*group + 4*(a/8) + a%4.  One round of permlane32 swaps brings
//             each block's other lane half to its own group; a fixed renaming
//             of registers then gives the columns in order.
// Either way lane b of group g ends with column b of D_g, i.e. row b of A B'.
// Each output element is its own dot product, so garbage in a padding lane's
// row only reaches that lane's row and column.
typedef float mma16_t __attribute__((ext_vector_type(16)));
typedef float mma32_t __attribute__((ext_vector_type(32)));
template <int NP>
struct MmaAcc {
    using type = mma16_t;
};
template <>
struct MmaAcc<32> {
    using type = mma32_t;
};
template <int NP>
using mma_t = typename MmaAcc<NP>::type;

// acc += A B' over columns k < K of the lane's rows a (of A) and b (of B)
template <int K>
__device__ __forceinline__ void mma_abt(mma16_t& acc, const float* a, const float* b)
{
#pragma unroll
    for (int k = 0; k < K; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x1f32(b[k], a[k], acc, 0, 0, 0);
}

template <int K>
__device__ __forceinline__ void mma_abt(mma32_t& acc, const float* a, const float* b)
{
#pragma unroll
    for (int k = 0; k < K; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x1f32(b[k], a[k], acc, 0, 0, 0);
}

__device__ __forceinline__ void swap_rows32(float& x, float& y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

__device__ __forceinline__ void swap_rows16(float& x, float& y)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

// r[c] = (A B')[lane][c] for c < NCOL, from an accumulator filled by mma_abt.
template <int NCOL>
__device__ __forceinline__ void mma_rows(const mma16_t& acc, float* r)
{
    static_assert(NCOL <= 16, "");
    float t[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) t[v] = acc[v];
    // rows 2-3 of quartets 0-1 <-> rows 0-1 of quartets 2-3
#pragma unroll
    for (int v = 0; v < 8; ++v) swap_rows32(t[v], t[v + 8]);
    // rows 1, 3 of quartets 0, 2 <-> rows 0, 2 of quartets 1, 3
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        swap_rows16(t[v], t[v + 4]);
        swap_rows16(t[v + 8], t[v + 12]);
    }
#pragma unroll
    for (int c = 0; c < NCOL; ++c) r[c] = t[c];
}

template <int NCOL>
__device__ __forceinline__ void mma_rows(const mma32_t& acc, float* r)
{
    static_assert(NCOL <= 32, "");
    float t[32];
#pragma unroll
    for (int v = 0; v < 32; ++v) t[v] = acc[v];
    // upper lane half of block 0 <-> lower lane half of block 1
#pragma unroll
    for (int v = 0; v < 16; ++v) swap_rows32(t[v], t[v + 16]);
    // column c: lane half (c/4)%2 of register quartet c/8
#pragma unroll
    for (int c = 0; c < NCOL; ++c) r[c] = t[(c % 8 < 4) ? 4 * (c / 8) + c % 4 : 16 + 4 * (c / 8) + c % 4];
}

// ------------------------------------------------------------------ in-place Gauss-Jordan

// Inverse of the K x K matrix whose row i is held by lane i of the group
// (rows beyond K are ignored), by Gauss-Jordan elimination without pivoting
// (the matrices are symmetric positive definite, whose pivots are the positive
// diagonal entries of their LDL' factor).  `bad` is set when a pivot is not
// positive or not finite (by gj_steps in the lane whose row gave the pivot, by
// gj_steps_lds in every lane; callers take it over the group); the elimination
// then continues with the bad pivot and the result is flagged, not repaired.
//
// Step j: every lane i != j subtracts A[i][j]/A[j][j] times row j and column j
// becomes the matching column of the inverse (the classical in-place form),
// but the pivot row is left unscaled: every row stays a multiple of its row of
// the classical form (row j by the factor A[j][j], its pivot), which every
// later step carries consistently, since it only adds multiples of the current
// pivot row to other rows with multipliers taken from those rows.  Each lane
// keeps the reciprocal of its own pivot and scales its row once, at the end
// (gj_finish).  Scaling the pivot row inside the step by a fused multiply-add
// with the multiplier (1/piv - 1) would round that multiplier in absolute
// terms, a relative error of up to 2^-24 * piv in the inverse's row.
template <int NP, int K, int J = 0>
__device__ __forceinline__ void gj_steps(float* a, int lane, float& mypiv, float& rinv)
{
    if constexpr (J < K) {
        float piv;
        if constexpr (NP == 16 || J < 16) {
            float lo = a[J];
            if constexpr (NP == 32) {
                float hi;
                dup_rows(a[J], lo, hi);
            }
            piv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(lo), 0x150 + (J & 15), 0xF, 0xF, false));
        } else {
            float lo, hi;
            dup_rows(a[J], lo, hi);
            piv = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(hi), 0x150 + (J & 15), 0xF, 0xF, false));
        }
        const float inv = __builtin_amdgcn_rcpf(piv);  // v_rcp_f32, 1 ulp
        const bool me = lane == J;
        mypiv = me ? piv : mypiv;
        const float f = a[J];
        const float g = me ? 0.0f : -(f * inv);
        float keep = a[J];
        if constexpr (NP == 16) {
            BcBs<(K < 16 ? K : 16)>::template run<J & 15>(a, g);
        } else {
            BcRow<32, K> src(a);
            axpyb<32, K, J>(a, src, g);
        }
        // column J of the inverse: -A[i][j]/piv off the pivot row; on it the unscaled 1
        a[J] = me ? 1.0f : -(keep * inv);
        rinv = me ? inv : rinv;
        gj_steps<NP, K, J + 1>(a, lane, mypiv, rinv);
    }
}

// The deferred scaling of gj_steps: row i times the reciprocal of its pivot.
template <int K>
__device__ __forceinline__ void gj_finish(float* a, float rinv)
{
#pragma unroll
    for (int c = 0; c < K; ++c) a[c] *= rinv;
}

// Each lane keeps the pivot of its own row's step and tests it once at the end.
template <int NP, int K>
__device__ __forceinline__ void gj_steps(float* a, int lane, bool& bad)
{
    float rinv = 1.0f, mypiv = 1.0f;
    gj_steps<NP, K, 0>(a, lane, mypiv, rinv);
    gj_finish<K>(a, rinv);
    bad |= !(mypiv > 0.0f) || !__builtin_isfinite(mypiv);
}

// The same elimination for 32-lane groups with the pivot rows passed through
// LDS instead of DPP: a 32-lane broadcast by DPP costs a permlane swap and a
// DPP multiply-add per column, here a step is a few float4 stores and loads and
// K plain multiply-adds.  The LDS round trip, not the arithmetic, bounds a
// step, so gj_lds_block(K) pivots share one: lanes J0 .. J0+BS-1 store their
// rows to the group's buffer `pr` (16-byte aligned, GJ_LDS_BLOCK rows of K
// rounded up to 4 floats), every lane reads them back, and before each of
// those pivots takes its step every lane applies the block's earlier steps to
// its copies of the later pivot rows, with the same multiply-adds their own
// lanes apply to them, so every row ends with the bits of one pivot row per
// round trip.  LDS accesses of one wave complete in order, and a group never
// spans two waves, so no barrier is needed.  Same arithmetic as gj_steps (the
// multiply-add a[c] + g * pivot_row[c] for every column, the pivot row left
// unscaled, each row scaled by its pivot's reciprocal at the end).
// Three rows per round trip measured fastest at n = 24 (the step 66.5 -> 59.3 us
// at B = 256, against 61.3 us with two and 60.9 with four); wider rows (n = 28)
// take two, where three would spill registers in the fused step.
constexpr int GJ_LDS_BLOCK = 3;  // the most rows any K takes (the buffers' size)
__host__ __device__ constexpr int gj_lds_block(int K) { return K > 24 ? 2 : GJ_LDS_BLOCK; }

template <int K, int BS, int J0 = 0>
__device__ __forceinline__ void gj_block_lds(float* a, int lane, bool& bad, float* pr, float& rinv)
{
    if constexpr (J0 < K) {
        constexpr int K4 = (K + 3) / 4, NB = (K - J0 < BS) ? K - J0 : BS;
        const int bl = lane - J0;
        if (bl >= 0 && bl < NB)
#pragma unroll
            for (int q = 0; q < K4; ++q) {
                float4 v;
                v.x = a[4 * q];
                v.y = 4 * q + 1 < K ? a[4 * q + 1] : 0.0f;
                v.z = 4 * q + 2 < K ? a[4 * q + 2] : 0.0f;
                v.w = 4 * q + 3 < K ? a[4 * q + 3] : 0.0f;
                reinterpret_cast<float4*>(pr)[bl * K4 + q] = v;
            }
        __builtin_amdgcn_wave_barrier();
        float rows[NB][4 * K4];
#pragma unroll
        for (int r = 0; r < NB; ++r)
#pragma unroll
            for (int q = 0; q < K4; ++q) {
                const float4 v = reinterpret_cast<const float4*>(pr)[r * K4 + q];
                rows[r][4 * q] = v.x;
                rows[r][4 * q + 1] = v.y;
                rows[r][4 * q + 2] = v.z;
                rows[r][4 * q + 3] = v.w;
            }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            const int J = J0 + r;
            const float piv = rows[r][J];
            bad |= !(piv > 0.0f) || !__builtin_isfinite(piv);
            const float inv = __builtin_amdgcn_rcpf(piv);  // v_rcp_f32, 1 ulp
            const bool me = lane == J;
            const float keep = a[J];
            const float g = me ? 0.0f : -(keep * inv);
#pragma unroll
            for (int c = 0; c < K; ++c) a[c] = __builtin_fmaf(rows[r][c], g, a[c]);
            a[J] = me ? 1.0f : -(keep * inv);
            rinv = me ? inv : rinv;
            // the block's later pivot rows take this step as their lanes do
#pragma unroll
            for (int r2 = r + 1; r2 < NB; ++r2) {
                const float k2 = rows[r2][J];
                const float g2 = -(k2 * inv);
#pragma unroll
                for (int c = 0; c < K; ++c) rows[r2][c] = __builtin_fmaf(rows[r][c], g2, rows[r2][c]);
                rows[r2][J] = -(k2 * inv);
            }
        }
        gj_block_lds<K, BS, J0 + BS>(a, lane, bad, pr, rinv);
    }
}

template <int K>
__device__ __forceinline__ void gj_steps_lds(float* a, int lane, bool& bad, float* pr)
{
    float rinv = 1.0f;
    gj_block_lds<K, gj_lds_block(K)>(a, lane, bad, pr, rinv);
    gj_finish<K>(a, rinv);
}

}  // namespace gato
