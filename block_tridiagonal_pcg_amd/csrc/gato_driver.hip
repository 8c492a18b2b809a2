// gato_driver.hip -- the SQP driver's per-iteration kernels around gato_sqp_step
// (include/gato_driver.h): the chain plant's QP at the current trajectory, and
// the selected step with the damping update.  Both are elementwise over knots
// and bound by their memory traffic; one lane per row of a knot's blocks.
#include "gato_driver.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

namespace gato {

struct ChainArgs {
    int d, N, B;
    float h, a, c, kappa, w_theta, w_omega, w_u;
};

// One thread per (solve, knot, state row i < n): row i of Q_k, A_k, B_k and the
// entries q_k[i], e_k[i]; rows i < m also write row i of R_k and r_k[i]; knot 0
// writes x0[i].  Rows of A_k for theta (i < d) are [e_i, h e_i]; rows for omega
// (i = d + j) are [h (-a cos(theta_j) e_j + kappa L_j), (1 - h c) e_j].
__global__ void k_chain_qp(ChainArgs g, const float* X, const float* U, const float* xi, const float* xr, float* Q,
                           float* q, float* R, float* r, float* A, float* Bu, float* e, float* x0)
{
    const int d = g.d, n = 2 * d, m = d, N = g.N;
    const size_t total = (size_t)g.B * N * n;
    for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (size_t)gridDim.x * blockDim.x) {
        const int i = (int)(t % n);
        const size_t bk = t / n;  // b * N + k
        const int k = (int)(bk % N);
        const size_t b = bk / N;
        const float* x = X + bk * n;
        const float w = i < d ? g.w_theta : g.w_omega;
        // Q_k row i, q_k[i] (every knot)
        float* Qr = Q + (bk * n + i) * n;
        for (int c = 0; c < n; ++c) Qr[c] = c == i ? w : 0.0f;
        q[bk * n + i] = w * (x[i] - xr[b * n + i]);
        if (k == 0) x0[b * n + i] = xi[b * n + i] - x[i];
        if (k == N - 1) continue;
        const size_t kd = b * (N - 1) + k;  // dynamics index
        const float* u = U + kd * m;
        float* Ar = A + (kd * n + i) * n;
        float* Br = Bu + (kd * n + i) * m;
        float f;
        if (i < d) {
            for (int c = 0; c < n; ++c) Ar[c] = c == i ? 1.0f : (c == d + i ? g.h : 0.0f);
            for (int c = 0; c < m; ++c) Br[c] = 0.0f;
            f = x[i] + g.h * x[d + i];
        } else {
            const int j = i - d;
            const float th = x[j];
            // (L theta)_j over the path graph with free ends
            const float lm = j > 0 ? 1.0f : 0.0f, lp = j + 1 < d ? 1.0f : 0.0f;
            const float lth = (j > 0 ? x[j - 1] : 0.0f) + (j + 1 < d ? x[j + 1] : 0.0f) - (lm + lp) * th;
            for (int c = 0; c < d; ++c) {
                const float lap = c == j ? -(lm + lp) : ((c == j - 1 || c == j + 1) ? 1.0f : 0.0f);
                Ar[c] = g.h * ((c == j ? -g.a * cosf(th) : 0.0f) + g.kappa * lap);
            }
            for (int c = 0; c < d; ++c) Ar[d + c] = c == j ? 1.0f - g.h * g.c : 0.0f;
            for (int c = 0; c < m; ++c) Br[c] = c == j ? g.h : 0.0f;
            const float acc = -g.a * sinf(th) - g.c * x[i] + g.kappa * lth + u[j];
            f = x[i] + g.h * acc;
        }
        e[kd * n + i] = f - X[(bk + 1) * n + i];
        if (i < m) {
            float* Rr = R + (kd * m + i) * m;
            for (int c = 0; c < m; ++c) Rr[c] = c == i ? g.w_u : 0.0f;
            r[kd * m + i] = g.w_u * u[i];
        }
    }
}

struct StepArgs {
    int n, m, N, B, n_alpha;
    float rho_min, rho_max;
    float alphas[GATO_MAX_ALPHA];
};

// One thread per entry of X and U (and per solve for rho).
__global__ void k_take_step(StepArgs g, const float* dz, const int32_t* best, float* X, float* U, float* rho)
{
    const int n = g.n, m = g.m, N = g.N;
    const size_t nx = (size_t)g.B * N * n, nu = (size_t)g.B * (N - 1) * m;
    const size_t per = (size_t)N * n + (size_t)(N - 1) * m;
    for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < nx + nu + g.B;
         t += (size_t)gridDim.x * blockDim.x) {
        if (t < nx + nu) {
            const bool isx = t < nx;
            const size_t o = isx ? t : t - nx;
            const int w = isx ? n : m;
            const size_t bk = o / w;
            const int i = (int)(o % w);
            const size_t b = isx ? bk / N : bk / (N - 1);
            const int k = (int)(isx ? bk % N : bk % (N - 1));
            const int s = best[b];
            const float a = (s >= 0 && s < g.n_alpha) ? g.alphas[s] : 0.0f;
            const float step = dz[b * per + (size_t)k * (n + m) + (isx ? i : n + i)];
            if (isx)
                X[t] += a * step;
            else
                U[o] += a * step;
        } else {
            const size_t b = t - nx - nu;
            const int s = best[b];
            const bool failed = !(s >= 0 && s < g.n_alpha);
            float v = rho[b];
            if (s == 0) v = fmaxf(v / 10.0f, g.rho_min);
            if (failed) v = fminf(v * 10.0f, g.rho_max);
            rho[b] = v;
        }
    }
}

static unsigned grid_for(size_t total)
{
    return (unsigned)std::max<size_t>(1, std::min<size_t>((total + 255) / 256, 8192));
}

}  // namespace gato

using namespace gato;

extern "C" {

int gato_chain_qp(const gato_dims_t* dims, const gato_chain_t* plant, const float* X, const float* U,
                  const float* x_init, const float* x_ref, float* Q, float* q, float* R, float* r, float* A,
                  float* Bu, float* e, float* x0, hipStream_t stream)
{
    if (dims == nullptr || plant == nullptr) return GATO_E_NULL;
    if (dims->B < 0 || dims->N < 2 || plant->dof < 1 || dims->n != 2 * plant->dof || dims->m != plant->dof)
        return GATO_E_DIMS;
    if (!(plant->h > 0.0f)) return GATO_E_PARAM;
    if (dims->B == 0) return GATO_OK;
    for (const void* p : {(const void*)X, (const void*)U, (const void*)x_init, (const void*)x_ref, (const void*)Q,
                          (const void*)q, (const void*)R, (const void*)r, (const void*)A, (const void*)Bu,
                          (const void*)e, (const void*)x0})
        if (p == nullptr) return GATO_E_NULL;
    ChainArgs g{plant->dof, dims->N, dims->B, plant->h, plant->a, plant->c, plant->kappa, plant->w_theta,
                plant->w_omega, plant->w_u};
    const size_t total = (size_t)dims->B * dims->N * dims->n;
    hipLaunchKernelGGL(k_chain_qp, dim3(grid_for(total)), dim3(256), 0, stream, g, X, U, x_init, x_ref, Q, q, R, r,
                       A, Bu, e, x0);
    return hipGetLastError() == hipSuccess ? GATO_OK : GATO_E_HIP;
}

int gato_take_step(const gato_dims_t* dims, const float* alphas_host, int32_t n_alpha, const float* dz,
                   const int32_t* best, float* X, float* U, float* rho, float rho_min, float rho_max,
                   hipStream_t stream)
{
    if (dims == nullptr || alphas_host == nullptr) return GATO_E_NULL;
    if (dims->B < 0 || dims->N < 1 || dims->n < 1 || dims->m < 1) return GATO_E_DIMS;
    if (n_alpha < 1 || n_alpha > GATO_MAX_ALPHA || !(rho_min > 0.0f) || !(rho_max >= rho_min)) return GATO_E_PARAM;
    if (dims->B == 0) return GATO_OK;
    if (dz == nullptr || best == nullptr || X == nullptr || rho == nullptr || (dims->N > 1 && U == nullptr))
        return GATO_E_NULL;
    StepArgs g{dims->n, dims->m, dims->N, dims->B, n_alpha, rho_min, rho_max, {}};
    for (int j = 0; j < n_alpha; ++j) g.alphas[j] = alphas_host[j];
    const size_t total = (size_t)dims->B * dims->N * dims->n + (size_t)dims->B * (dims->N - 1) * dims->m + dims->B;
    hipLaunchKernelGGL(k_take_step, dim3(grid_for(total)), dim3(256), 0, stream, g, dz, best, X, U, rho);
    return hipGetLastError() == hipSuccess ? GATO_OK : GATO_E_HIP;
}

}  // extern "C"
