// gato_cr.hip -- stage 2 by block cyclic reduction (gato_cr_solve, and the
// long-horizon solve of gato_sqp_step while its log-depth pays).
//
// Kernels (one workgroup per solve unless noted):
//   k_cr_res     every knot of the solve held in registers and LDS (n <= 16, N <= 128).
//   k_cr_res_ref the same followed by a pass of KKT iterative refinement on its factors.
//   k_nd_reduce, k_cr_res<VIRT>, k_nd_back
//                nested dissection for n <= 16, N > 128: chunk interiors eliminated
//                in order, the chunks' boundary system reduced cyclically, then
//                the interiors back-substituted (the two chunk kernels spread a
//                solve's chunks over ND_SPLIT workgroups).
//   k_cr         any horizon and shape, the reduced rows kept in the workspace.
#include "gato_internal.h"
#include "gato_cr.h"

#include <algorithm>

namespace gato {

// ------------------------------------------------------------------ stage 2, cyclic reduction

// One workgroup per solve; up to 64 lane groups (32 for n > 16, whose rows
// are twice as wide) share the eliminations of each level.  A horizon of N
// knots has at most ceil(N/2) eliminations per level, so shorter horizons
// get fewer waves.
template <class SH>
struct CrLaunch {
    static constexpr int MAXT = SH::NP == 16 ? 1024 : 512;
    static int threads(int N)
    {
        const int cap = MAXT / SH::NP;
        const int want = (N + 1) / 2;
        const int groups = want < 1 ? 1 : (want < cap ? want : cap);
        return ((groups + SH::KPW - 1) / SH::KPW) * 64;
    }
};

template <class SH>
__global__ __launch_bounds__(CrLaunch<SH>::MAXT) void k_cr(Params p)
{
    cr_solve<SH>(p, blockIdx.x);
}

// Horizons whose knots fit in one workgroup's registers (n <= 16, N <= 128):
// two knots per lane group, W blocks exchanged through LDS.
template <class SH>
__global__ __launch_bounds__(1024) void k_cr_res(Params p)
{
    cr_resident<SH>(p, blockIdx.x);
}

// The same, followed inside the kernel by one pass of KKT iterative refinement
// that reuses the solve's factors (gato_sqp_step's default on these horizons).
template <class SH>
__global__ __launch_bounds__(1024) void k_cr_res_ref(Params p)
{
    cr_resident<SH, false, true>(p, blockIdx.x);
}

// Nested dissection (n <= 16, N > 128): the chunk kernels take ND_SPLIT
// workgroups of ND_GPW lane groups per solve, the boundary system one
// workgroup of 64 lane groups.
template <class SH>
__global__ __launch_bounds__(ND_GPW * 16) void k_nd_reduce(Params p)
{
    nd_reduce<SH>(p, blockIdx.x);
}

template <class SH>
__global__ __launch_bounds__(1024) void k_cr_res_virt(Params p)
{
    cr_resident<SH, true>(p, blockIdx.x);
}

template <class SH>
__global__ __launch_bounds__(ND_GPW * 16) void k_nd_back(Params p)
{
    nd_back<SH>(p, blockIdx.x);
}

template <class SH>
static bool cr_resident(int N, bool stream)
{
    if constexpr (SH::NP == 16) return N <= 2 * CrResLds<SH>::MAXG && !stream;
    return false;
}

template <class SH>
static hipError_t cr_launch_shape(const Params& p, hipStream_t st)
{
    if constexpr (SH::NP == 16) {
        if (cr_resident<SH>(p.N, p.cr_stream != 0)) {
            const int groups = (p.N + 1) / 2;
            hipLaunchKernelGGL((k_cr_res<SH>), dim3(p.B), dim3(((groups + SH::KPW - 1) / SH::KPW) * 64), 0, st, p);
            return hipGetLastError();
        }
        if (!p.cr_stream) {  // N > 128: nested dissection
            static_assert(2 * ND_CHUNKS == 2 * CrResLds<SH>::MAXG, "boundary system = one resident workgroup");
            const dim3 chunks(p.B, ND_SPLIT), blk(ND_GPW * SH::NP);
            hipLaunchKernelGGL((k_nd_reduce<SH>), chunks, blk, 0, st, p);
            hipLaunchKernelGGL((k_cr_res_virt<SH>), dim3(p.B), dim3(ND_CHUNKS * SH::NP), 0, st, p);
            hipLaunchKernelGGL((k_nd_back<SH>), chunks, blk, 0, st, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_cr<SH>), dim3(p.B), dim3(CrLaunch<SH>::threads(p.N)), 0, st, p);
    return hipGetLastError();
}

template <class SH>
static hipError_t cr_launch_refined_shape(const Params& p, hipStream_t st)
{
    if constexpr (SH::NP == 16) {
        if (cr_resident<SH>(p.N, p.cr_stream != 0)) {
            const int groups = (p.N + 1) / 2;
            hipLaunchKernelGGL((k_cr_res_ref<SH>), dim3(p.B), dim3(((groups + SH::KPW - 1) / SH::KPW) * 64), 0, st,
                               p);
            return hipGetLastError();
        }
    }
    return hipErrorInvalidValue;
}

template <class F>
static int with_cr_shape(int n, int m, F&& f)
{
#define GATO_CR_SHAPE(n_, m_) \
    if (n == n_ && m == m_) return f(Shape<n_, m_>{});
    GATO_FOR_SHAPES(GATO_CR_SHAPE)
#undef GATO_CR_SHAPE
    return -1;
}

hipError_t cr_launch(const Params& p, hipStream_t st)
{
    hipError_t e = hipErrorInvalidValue;
    with_cr_shape(p.n, p.m, [&](auto sh) {
        e = cr_launch_shape<decltype(sh)>(p, st);
        return 0;
    });
    return e;
}

bool cr_refines_inside(const gato_dims_t* d, bool stream)
{
    return d->n <= 16 && d->N <= 128 && !stream;
}

hipError_t cr_launch_refined(const Params& p, hipStream_t st)
{
    hipError_t e = hipErrorInvalidValue;
    with_cr_shape(p.n, p.m, [&](auto sh) {
        e = cr_launch_refined_shape<decltype(sh)>(p, st);
        return 0;
    });
    return e;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Cyclic reduction: one row [L | U | gamma | D] per knot row, padded to float4s.
static size_t cr_row_floats(int n) { return (size_t)(3 * n + 1 + 3) / 4 * 4; }

size_t cr_ws_bytes(const gato_dims_t* d)
{
    // the largest of the layouts: the streaming kernel's rows (B N n W), the
    // resident kernel's parked rows (B ceil(N/2) n 16) with, for its refinement
    // pass, the even knots' as many and q' and r' (B N (n + m)), and the nested
    // dissection's (the interior
    // knots' factors, the boundary system's rows and its parked rows)
    const size_t B = d->B, N = d->N, n = d->n, W = cr_row_floats(d->n);
    const size_t stream = B * N * n * W;
    const size_t nd = B * (N * nd_fac_floats(d->n) + 2 * ND_CHUNKS * n * W) + B * ND_CHUNKS * n * 16;
    const size_t ref = 2 * B * ((N + 1) / 2) * n * 16 + B * N * (n + d->m);
    return align256(std::max({stream, nd, ref}) * sizeof(float));
}

bool cr_reads_lower(const gato_dims_t* d, bool stream)
{
    return !(d->n <= 16 && !stream);
}

// The long-horizon solve of gato_sqp_step, chosen by a cost model measured on
// MI355X.  Block Thomas walks the knots in order: about 2.7 us per knot
// whatever the batch (n <= 16; 6.9 us with 32-lane groups, n > 16) until its
// one lane group per solve fills the chip, about 1.5 ns per knot and solve
// beyond (5.6 ns for n > 16).  Cyclic reduction is log-depth but does more
// arithmetic: about 0.15 us + 1.05 ns per knot per solve with the
// register-resident kernel (N <= 128, n <= 16), 0.18 us + 1.9 ns per knot per
// solve with the nested dissection (N > 128, n <= 16) and 17 ns per knot and
// solve with the streaming kernel (n > 16), once its batch fills the chip.
// Cyclic reduction is taken while its batch time stays below block Thomas's
// (the n <= 16 constants are from n = 14, the n > 16 ones from n = 24).
// With the refinement pass (the step's default) the register-resident kernel
// refines on its own factors while block Thomas solves twice, so there the
// whole refined steps are compared instead, as measured (workload-3 data,
// N = 65 and 128, B up to 3072): about B (0.220 + 0.00363 N) us with the
// reduction against 3.6 N + 0.00465 N B us with block Thomas.  Elsewhere both
// solvers repeat their solve for the pass and the comparison of the solves
// stands.
bool cr_preferred(const gato_dims_t* d, bool refine)
{
    const bool narrow = d->n <= 16;
    if (refine && narrow && d->N <= 2 * ND_CHUNKS)
        return d->B * (0.220 + 0.00363 * d->N) < 3.6 * d->N + 0.00465 * d->N * d->B;
    const double per_solve_us =
        narrow ? (d->N <= 2 * ND_CHUNKS ? 0.15 + 0.00105 * d->N : 0.18 + 0.0019 * d->N) : 0.017 * d->N;
    const bool wide = d->n > 16;  // 32-lane groups
    const double thomas_us = std::max((wide ? 6.9 : 2.7) * d->N, (wide ? 0.0056 : 0.0015) * d->N * d->B);
    return d->B * per_solve_us < thomas_us;
}

}  // namespace gato
