"""fp64 CPU oracle for the batched SQP-step linear-algebra core (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product.

The arithmetic lives in ``gato_oracle.c`` (plain C, double precision); this
module only builds it with gcc, marshals numpy arrays and names the outputs.
"""
from .ref import (  # noqa: F401
    build,
    load,
    num_threads,
    set_num_threads,
    CFLAGS,
    form_schur,
    pcg_solve,
    merit_eval,
    sqp_step,
    direct_solve,
    cyclic_plan,
    recover,
    FLAG_Q_NOT_SPD,
    FLAG_R_NOT_SPD,
    FLAG_S_NOT_SPD,
    FLAG_PCG_MAXITER,
    FLAG_PCG_BREAKDOWN,
    FLAG_LS_FAILED,
    FLAG_NONFINITE,
)
