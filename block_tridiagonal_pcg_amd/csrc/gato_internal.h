// gato_internal.h -- host-side interface between the library's translation
// units: gato.hip (formation, PCG, block Thomas, merit, the C ABI) and
// gato_cr.hip (block cyclic reduction).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "gato.h"

// (n, m) of the shapes the library has kernels for: those of the configurations
// the benchmark and tests use, n = m = 1 for hand-checkable examples, and
// (28, 14), the widest whose fused step fits a workgroup's LDS, so that
// gato_sqp_step can serve any n <= 28, m <= 14 by padding.
#define GATO_FOR_SHAPES(X) X(14, 7) X(12, 6) X(24, 12) X(4, 2) X(1, 1) X(28, 14)

namespace gato {

struct Params;

// Workspace of gato_cr_solve: one float4-padded row [L | U | gamma | D] per
// knot row of every solve, 256-byte aligned size.
size_t cr_ws_bytes(const gato_dims_t* d);

// Launches the cyclic reduction for p (shape p.n x p.m, which must be one this
// build has kernels for): the register-resident kernel or the nested
// dissection where they apply and p.cr_stream is 0, else the streaming one.
hipError_t cr_launch(const Params& p, hipStream_t st);

// Whether the cyclic reduction cr_launch runs for these dimensions reads the
// lower blocks S_{k,k-1} (the streaming kernel does, and runs for n > 16 or
// when `stream` asks for it; the register-resident kernel and the nested
// dissection read the upper blocks only).
bool cr_reads_lower(const gato_dims_t* d, bool stream);

// Whether the cyclic reduction for these dimensions runs the refinement pass
// inside its kernel (cr_launch_refined): the register-resident kernel, n <= 16
// and N <= 128, unless `stream` asks for the streaming one.
bool cr_refines_inside(const gato_dims_t* d, bool stream);

// The register-resident cyclic reduction followed, in the same kernel, by one
// pass of KKT iterative refinement (the problem data, S, gamma, Q~^-1 and R^-1
// of p; lambda and dz are the refined ones); only where cr_refines_inside.
hipError_t cr_launch_refined(const Params& p, hipStream_t st);

// Whether gato_sqp_step takes cyclic reduction rather than block Thomas
// beyond the fused horizons, by the measured cost model of the step with
// (refine) or without its refinement pass.
bool cr_preferred(const gato_dims_t* d, bool refine);

}  // namespace gato
