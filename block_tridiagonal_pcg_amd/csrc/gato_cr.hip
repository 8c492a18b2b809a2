// gato_cr.hip -- stage 2 by block cyclic reduction (gato_cr_solve, and the
// long-horizon solve of gato_sqp_step while its log-depth pays).
//
// Kernels (one workgroup per solve):
//   k_cr_res  every knot of the solve held in registers and LDS (n <= 16, N <= 128).
//   k_cr      any horizon, the reduced rows kept in the workspace.
#include "gato_internal.h"
#include "gato_cr.h"

#include <cstdlib>
#include <cstring>

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
        int cap = MAXT / SH::NP;
        if (const char* env = std::getenv("GATO_CR_GROUPS")) {  // lane groups per workgroup (measurements)
            const int gr = std::atoi(env);
            if (gr >= 1 && gr < cap) cap = gr;
        }
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

static bool cr_streaming_forced()  // GATO_CR_VARIANT=stream: the streaming kernel for every N (measurements)
{
    const char* env = std::getenv("GATO_CR_VARIANT");
    return env && std::strcmp(env, "stream") == 0;
}

template <class SH>
static bool cr_resident(int N)
{
    if constexpr (SH::NP == 16) return N <= 2 * CrResLds<SH>::MAXG && !cr_streaming_forced();
    return false;
}

template <class SH>
static hipError_t cr_launch_shape(const Params& p, hipStream_t st)
{
    if constexpr (SH::NP == 16) {
        if (cr_resident<SH>(p.N)) {
            const int groups = (p.N + 1) / 2;
            hipLaunchKernelGGL((k_cr_res<SH>), dim3(p.B), dim3(((groups + SH::KPW - 1) / SH::KPW) * 64), 0, st, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_cr<SH>), dim3(p.B), dim3(CrLaunch<SH>::threads(p.N)), 0, st, p);
    return hipGetLastError();
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

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Cyclic reduction: one row [L | U | gamma | D] per knot row, padded to float4s.
static size_t cr_row_floats(int n) { return (size_t)(3 * n + 1 + 3) / 4 * 4; }

size_t cr_ws_bytes(const gato_dims_t* d)
{
    const size_t B = d->B, N = d->N, n = d->n;
    return align256(B * N * n * cr_row_floats(d->n) * sizeof(float));
}

// The long-horizon solve of gato_sqp_step, chosen by a cost model measured on
// MI355X (knots n = 14): block Thomas walks the knots in order, about 3.0 us
// per knot whatever the batch until its one lane group per solve fills the
// chip (about 1.6 ns per knot and solve beyond); cyclic reduction is
// log-depth but does twice the arithmetic, about 0.35 us per solve with the
// register-resident kernel (N <= 128, n <= 16) and 4.3 ns per knot and solve
// with the streaming one once the batch fills the chip.  Cyclic reduction is
// taken while its batch time stays below the Thomas walk's latency.
// GATO_LONG_SOLVE=thomas or =cr forces either (for measurements).
bool cr_preferred(const gato_dims_t* d)
{
    const bool resident = with_cr_shape(d->n, d->m, [&](auto sh) { return cr_resident<decltype(sh)>(d->N) ? 1 : 0; }) == 1;
    if (const char* env = std::getenv("GATO_LONG_SOLVE")) {
        if (std::strcmp(env, "thomas") == 0) return false;
        if (std::strcmp(env, "cr") == 0) return true;
    }
    const double thomas_us = 3.0 * d->N;
    const double cr_us = d->B * (resident ? 0.35 : 0.0043 * d->N);
    return cr_us < thomas_us;
}

}  // namespace gato
