#!/usr/bin/env python3
"""Throughput of one SQP iteration's linear-algebra core on one MI355X.

A step is gato_sqp_step over the whole batch: form S, gamma and the stair
preconditioner, PCG to eps = 1e-6, recover dz, merit at 8 step sizes and
select (GATO paper Sec. III, Fig. 2 steps a-c), cold-started: every timed step
starts from its own zeroed lambda buffer, so no step reuses another step's
solution.  Inputs (the problem data and the zero starting points) are seeded
synthetic batches (block_tridiagonal_pcg_amd.synth) already resident in device
memory when the timed region starts; the timed region is the K launches alone,
and HIP events on the launch stream around it give the kernel's average time.

Prints one JSON line.  Options: --steps K --warmup W --gpus N (N must be 1)
--config C --batch B --horizon N (the configuration's generators at another
horizon) --refine on|off --no-cpu-baseline.  Every run also times a 256 MiB
device copy (its rate is reported beside the published HBM peak; under the
profiler it is the reference kernel for scaling byte counters) and the K steps
once more one by one (median and 90th percentile).  Study modes, each one JSON
line instead of the step: --merit-variants, --sqp-driver, --solver-sweep, --step-sweep.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
EPS = 1e-6
MU = 1.0
CAPS = {1: 200, 2: 200, 3: 200, 4: 200, 5: 2000}
KERNEL = "k_sqp_fused"

# Timings the GATO pages give for the iiwa14-shaped horizon (n = 14, m = 7, N = 64) on other
# hardware (GATO docs, "Merit launch timing": the RTX 5090 table, the MPS-limited tables and the
# Jetson AGX Orin sweep of October 24).  They time whole nonlinear SQP solves with rigid-body
# dynamics and rollouts, not this LQ step: context printed beside the measurement, never a ratio.
PAGES_CONTEXT = {
    "note": "the pages' timings of whole nonlinear SQP solves on other hardware; context, not a target",
    "rtx5090_merit_launch_us_64_threads": {"B1": 33, "B8": 72, "B16": 119},
    "rtx5090_two_iteration_solve_ms_64_threads": {"B1": 2.273, "B8": 2.874, "B16": 3.057},
    "rtx5090_10pct_sms_merit_launch_us_64_threads": {"B1": 63, "B8": 289, "B16": 547},
    "jetson_orin_40W_linsys_ms_per_solve_B1": {"cold": 12.32, "warm": [15.45, 16.34],
                                               "note": "plant and N not stated on the page"},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--batch", type=int, default=128)
    ap.add_argument("--horizon", type=int, default=None, help="override the configuration's N")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--refine", choices=("on", "off"), default="on",
                    help="the KKT refinement pass after a direct solve (on: the library's default; "
                         "off: gato_sqp_step_opts with refine = 0, for comparison)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile-copy", action="store_true", help="accepted for old command lines; the copy always runs")
    ap.add_argument("--merit-variants", action="store_true",
                    help="instead of the step: time the merit call's launch variants (one JSON line)")
    ap.add_argument("--sqp-driver", action="store_true",
                    help="instead of the step: time the multi-iteration SQP driver on the pendulum-chain plant")
    ap.add_argument("--solver-sweep", action="store_true",
                    help="instead of the step: time the block Thomas and cyclic-reduction solves over horizons "
                         "and batch sizes (the measurements behind gato_sqp_step's switch)")
    ap.add_argument("--step-sweep", action="store_true",
                    help="instead of the step: time the whole step (refinement on) with cyclic reduction and "
                         "with block Thomas over horizons and batch sizes, beside gato_step_solver's choice")
    return ap.parse_args()


# ---------------------------------------------------------------- algorithmic work


def form_flops(n, m, N):
    """Dense-block operation count of stage 1 per solve.

    Per knot: SPD inverses of Q~ (n^3) and R (m^3) [Cholesky n^3/3 + triangular
    inverse n^3/3 + product n^3/3]; A Q~^-1 and A Q~^-1 A' (2 n^3 each); B R^-1 (2 n m^2)
    and B R^-1 B' (2 n^2 m); D^-1 (n^3); -D_k^-1 S_{k,k+1} D_{k+1}^-1 (4 n^3); gamma
    (Q~^-1 q, A Q~^-1 q, B R^-1 r: 2 n^2 + 2 n^2 + 2 n m) and the D sum (2 n^2).
    """
    per_dyn = 2 * n ** 3 + 2 * n ** 3 + 2 * n * m * m + 2 * n * n * m + m ** 3 + 4 * n ** 3 + 4 * n * n + 2 * n * m
    per_knot = n ** 3 + n ** 3 + 2 * n * n
    return N * per_knot + (N - 1) * per_dyn


def pcg_iter_flops(n, N):
    """Per PCG iteration per solve: S p and Phi^-1 r over (3N-2) n x n blocks (2 flops per
    entry each), three dot products and three axpys over N n entries."""
    return 2 * 2 * (3 * N - 2) * n * n + 3 * 2 * N * n + 3 * 2 * N * n


def pcg_iter_bytes(n, N):
    """Unique fp32 entries of S and Phi^-1 read per iteration per solve (symmetric diagonal
    blocks counted once per triangle, off-diagonal blocks once)."""
    return 4 * 2 * (N * n * (n + 1) // 2 + (N - 1) * n * n)


def direct_flops(n, m, N):
    """Block elimination per solve: per knot the Gauss-Jordan inverse of H_k (2 n^3) and the
    back substitution (two n x n products with a vector, 4 n^2); per dynamics step
    T = S_{k,k-1} H^-1 and T S_{k-1,k} (2 n^3 each) and the right-hand side update."""
    return N * (2 * n ** 3 + 4 * n * n + n) + (N - 1) * (4 * n ** 3 + 3 * n * n)


def cr_flops(n, N):
    """Block cyclic reduction per solve, level by level: each eliminated knot factors its
    pivot block (n^3/3) and solves it against [L U gamma] (2n+1 columns of n^2); each kept
    knot takes W2'W2 and W2'w3 from its left neighbour (2 n^3 + 2 n^2) and W1'W1, W1'W2,
    W1'w3 from its right one (4 n^3 + 2 n^2); the back substitution costs two products with
    a vector and a triangular solve (5 n^2) per eliminated knot; the last knot is factored
    and solved alone (n^3/3 + 2 n^2)."""
    f = 0.0
    s = 1
    while s < N:
        for j in range(s, N, 2 * s):
            f += n ** 3 / 3 + (2 * n + 1) * n * n + 5 * n * n
            f += 2 * n ** 3 + 2 * n * n  # into the kept knot j - s
            if j + s < N:
                f += 4 * n ** 3 + 2 * n * n  # into the kept knot j + s
        s *= 2
    return f + n ** 3 / 3 + 2 * n * n


def recover_flops(n, m, N):
    return N * 2 * n * n + (N - 1) * (2 * n * n + 2 * n * m + 2 * m * m) + 4 * N * n


def merit_flops(n, m, N, n_alpha):
    """Per solve: Q dx, R du, A dx + B du computed once per knot (2 flops per entry),
    the linear/quadratic terms, and per step size |e + a d| (3 per entry) plus the sums."""
    per_knot = 2 * n * n + 2 * m * m + 2 * n * n + 2 * n * m + 4 * n + 4 * m
    return N * per_knot + (n_alpha + 1) * (N * 3 * n + 5 * N)


def input_bytes(n, m, N):
    return 4 * (N * n * n + N * n + (N - 1) * (m * m + m + n * n + n * m + n) + n)


def output_bytes(n, m, N, n_alpha):
    """lambda, dz and the merits per solve, plus merit0, best, iters, relres and flags."""
    return 4 * (N * n + N * n + (N - 1) * m + n_alpha + 5)


# ---------------------------------------------------------------- measured traffic


# The translation unit that holds the fused step kernel (the cyclic reduction's
# own sources, gato_cr.h and gato_cr.hip, do not enter it).
FUSED_SOURCES = ("block_tridiagonal_pcg_amd/csrc/gato.hip", "block_tridiagonal_pcg_amd/csrc/gato_stages.h",
                 "block_tridiagonal_pcg_amd/csrc/gato_dev.h", "block_tridiagonal_pcg_amd/csrc/dpp_asm.inc",
                 "block_tridiagonal_pcg_amd/csrc/gato_internal.h", "include/gato.h")


def _code_only(text):
    """C/C++ source without its comments and with whitespace collapsed: what the
    compiler sees (the sources hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(read=None):
    """Digest of the fused kernel's sources, comments excluded (a comment cannot
    change the kernel the counters were taken on)."""
    read = read or (lambda f: open(os.path.join(ROOT, f)).read())
    h = hashlib.sha256()
    for f in FUSED_SOURCES:
        h.update(_code_only(read(f)).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources and this workload; else None."""
    path = os.path.join(ROOT, "profiles", "k_sqp_fused_cfg3_B128_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != source_digest() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------- CPU baseline


def cpu_model():
    """The host CPU's model name, as the kernel reports it."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def _median_time(fn, reps):
    import statistics

    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts), ts


def cpu_baseline(batch, n_alpha, seconds):
    """The oracle as it stands, on this host's cores: the whole step (form, PCG,
    recovery, merit, selection; same eps and cap) over the timed batch on all the
    threads OpenMP gives it, then on one thread over a sample of the batch, then its
    three stages alone; medians of repeated runs.  About `seconds` of wall time."""
    import numpy as np

    import oracle

    al = np.array([2.0 ** -i for i in range(n_alpha)])
    cap = CAPS[batch["cid"]]
    B = batch["dims"][3]
    args = [batch[f] for f in ("Q", "q", "R", "r", "A", "Bu", "e", "x0")]
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    first = oracle.sqp_step(*args, None, EPS, cap, al, MU)
    one = time.perf_counter() - t0
    # all threads: the whole batch, at least 5 repeats, about half the budget
    reps = max(5, min(2000, int(0.5 * seconds / max(one, 1e-6))))
    med, ts = _median_time(lambda: oracle.sqp_step(*args, None, EPS, cap, al, MU), reps)
    # one thread: a leading sample of the batch sized for ~30 % of the budget over 5 repeats
    per_solve_1 = one * threads / B  # assumes the threads scale; only sizes the sample
    b1 = int(max(1, min(B, 0.3 * seconds / 5 / max(per_solve_1, 1e-9))))
    sub = [x[:b1] for x in args]
    oracle.set_num_threads(1)
    try:
        med1, _ = _median_time(lambda: oracle.sqp_step(*sub, None, EPS, cap, al, MU), 5)
    finally:
        oracle.set_num_threads(threads)
    # the stages alone (all threads, whole batch, median of 3)
    f = oracle.form_schur(*args)
    t_form, _ = _median_time(lambda: oracle.form_schur(*args), 3)
    t_pcg, _ = _median_time(lambda: oracle.pcg_solve(f["S"], f["Pinv"], f["gamma"], f["Qinv"], f["Rinv"],
                                                     batch["A"], batch["Bu"], batch["q"], batch["r"], EPS, cap), 3)
    t_mer, _ = _median_time(lambda: oracle.merit_eval(*args, first["dz"], al, MU), 3)
    rec = {"value": B / med, "unit": "solves/s", "cores": threads, "kind": "oracle",
           "sample": "the full %d-solve batch of the timed workload, median of %d repeats (%.1f s), fp64, "
                     "OpenMP over solves" % (B, reps, sum(ts)),
           "one_core": {"value": b1 / med1, "unit": "solves/s", "cores": 1,
                        "sample": "solves 0..%d of the batch, median of 5 repeats" % (b1 - 1)},
           "stage_us": {"schur_us": t_form * 1e6, "linsys_us": t_pcg * 1e6, "merit_us": t_mer * 1e6,
                        "note": "whole batch, all threads, median of 3; linsys is PCG plus the recovery"},
           "cpu_model": cpu_model(),
           "compiler": "gcc " + " ".join(oracle.CFLAGS),
           "statistic": "median"}
    return rec, first


def iters_summary(x):
    import numpy as np

    return {"min": int(x.min()), "median": float(np.median(x)), "max": int(x.max())}


def exact_step(batch, n_alpha):
    """The oracle's exact step on the batch: lambda by block Cholesky of S, then dz and
    the merits (the reference for the direct solves)."""
    import numpy as np

    import oracle

    ins = [batch[f] for f in ("Q", "q", "R", "r", "A", "Bu", "e", "x0")]
    al = np.array([2.0 ** -i for i in range(n_alpha)])
    form = oracle.form_schur(*ins)
    lam = oracle.direct_solve(form["S"], form["gamma"])["lam"]
    dz = oracle.recover(form["Qinv"], form["Rinv"], batch["A"], batch["Bu"], batch["q"], batch["r"], lam)
    mer = oracle.merit_eval(*ins, dz, al, MU)
    return {"dz": dz, "merit": mer["merit"], "best": mer["best"]}


def rel_err_rows(g, o):
    """Per-solve relative 2-norm error of g against o (rows = solves)."""
    import numpy as np

    g = np.asarray(g, dtype=np.float64).reshape(len(o), -1)
    o = np.asarray(o, dtype=np.float64).reshape(len(o), -1)
    return np.linalg.norm(g - o, axis=1) / np.maximum(np.linalg.norm(o, axis=1), 1e-300)


# ---------------------------------------------------------------- merit launch variants


def _hip():
    """The HIP runtime this process already loaded (torch's and libgato's), for CU-masked streams."""
    import ctypes

    path = None
    for line in open("/proc/self/maps"):
        if "libamdhip64" in line:
            path = line.split()[-1]
            break
    hip = ctypes.CDLL(path or "libamdhip64.so")
    V, U, P = ctypes.c_void_p, ctypes.c_uint32, ctypes.POINTER(ctypes.c_void_p)
    hip.hipExtStreamCreateWithCUMask.argtypes = [P, U, ctypes.POINTER(U)]
    hip.hipStreamDestroy.argtypes = [V]
    hip.hipEventCreate.argtypes = [P]
    hip.hipEventRecord.argtypes = [V, V]
    hip.hipEventSynchronize.argtypes = [V]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), V, V]
    hip.hipEventDestroy.argtypes = [V]
    return hip


def merit_variants(a):
    """Device time of gato_merit_eval per launch for each launch variant: the fused per-knot
    kernel and the candidate-parallel one, at workgroup sizes 64..1024, on the whole GPU and
    on streams restricted to fewer CUs (the few-SM analogue of the pages' MPS throttle)."""
    import ctypes

    import torch

    from block_tridiagonal_pcg_amd import ops, synth

    torch.cuda.set_device(0)
    hip = _hip()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    rows = []
    for B in (1, 16, 128):
        batch = synth.make_batch(a.config, B)
        dims = batch["dims"]
        dev = ops.to_device(batch)
        out = ops.alloc_outputs(dims, 8)
        ws = ops.workspace_for(dims, 8)
        ops.gato_sqp_step(dims, *[dev[f] for f in synth.FIELDS], None, EPS, CAPS[a.config], synth.ALPHAS, MU,
                          out["lam"], out["dz"], out["merit"], out["merit0"], out["best"], out["iters"],
                          out["relres"], out["flags"], workspace=ws)
        torch.cuda.synchronize()
        for cus in sorted({8, 32, 128, n_cu}):
            words = (n_cu + 31) // 32
            mask = (ctypes.c_uint32 * words)(*[
                sum(1 << b for b in range(32) if 32 * w + b < cus) for w in range(words)])
            st = ctypes.c_void_p()
            if hip.hipExtStreamCreateWithCUMask(ctypes.byref(st), words, mask) != 0:
                raise RuntimeError("hipExtStreamCreateWithCUMask failed")
            e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
            hip.hipEventCreate(ctypes.byref(e0))
            hip.hipEventCreate(ctypes.byref(e1))
            for variant in (ops.MERIT_PER_KNOT, ops.MERIT_PER_CANDIDATE):
                for waves in (1, 2, 4, 8, 16):
                    call = lambda: ops.gato_merit_eval(dims, *[dev[f] for f in synth.FIELDS], out["dz"],  # noqa
                                                       synth.ALPHAS, MU, out["merit"], out["merit0"], out["best"],
                                                       out["flags"], stream=st.value, variant=variant, waves=waves)
                    for _ in range(3):
                        call()
                    reps = 20
                    hip.hipEventRecord(e0, st)
                    for _ in range(reps):
                        call()
                    hip.hipEventRecord(e1, st)
                    hip.hipEventSynchronize(e1)
                    ms = ctypes.c_float()
                    hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1)
                    rows.append({"B": B, "cus": cus, "variant": ["fused", "candidate"][variant], "threads": 64 * waves,
                                 "us": ms.value * 1e3 / reps})
            hip.hipEventDestroy(e0)
            hip.hipEventDestroy(e1)
            hip.hipStreamDestroy(st)
    print(json.dumps({"study": "merit launch variants", "workload": synth.CONFIGS[a.config].name,
                      "unit": "us per launch", "rows": rows}))


# ---------------------------------------------------------------- SQP driver


def sqp_driver(a, iters=10, N=64, dof=7):
    """SQP iterations per second of the whole driver loop (plant linearisation on the
    device, gato_sqp_step, step and damping update) on the 7-DoF chain, and the fp64
    reference driver on the host for a sample of the batch."""
    import numpy as np
    import torch

    from block_tridiagonal_pcg_amd import driver, synth

    torch.cuda.set_device(0)
    P = synth.Chain(dof)
    B = a.batch
    xi, xr, rho = synth.chain_seed(P, B)
    driver.solve(P, xi, xr, rho, N, 2, record=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = driver.solve(P, xi, xr, rho, N, iters, record=False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    again = driver.solve(P, xi, xr, rho, N, iters, step_events=True)
    hist = again["history"]
    # the same iterations with one iteration captured in a HIP graph and replayed
    driver.solve(P, xi, xr, rho, N, 2, record=False, graph=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gres = driver.solve(P, xi, xr, rho, N, iters, record=False, graph=True)
    torch.cuda.synchronize()
    wall_graph = time.perf_counter() - t0
    rec = {"study": "SQP driver", "plant": "pendulum chain, %d DoF (n=%d, m=%d)" % (dof, P.n, P.m), "N": N, "B": B,
           "iterations": iters, "ms_per_iteration": wall / iters * 1e3,
           "solve_iterations_per_s": B * iters / wall,
           "graph_ms_per_iteration": wall_graph / iters * 1e3,
           "graph_solve_iterations_per_s": B * iters / wall_graph,
           "graph_replay_ms_per_iteration": gres["replay_us"] / 1e3,
           "graph_replay_solve_iterations_per_s": B / (gres["replay_us"] * 1e-6),
           "graph_note": "first iteration eager, then one captured iteration replayed; graph_ms_per_iteration "
                         "is the wall time including the eager iteration and the capture, graph_replay_* the "
                         "replays alone (HIP events)",
           "defect_max_first": float(hist[0]["defect"].max()), "defect_max_last": float(hist[-1]["defect"].max()),
           "pcg_iters_per_iteration": [int(np.median(h["iters"])) for h in hist],
           "sqp_step_us_per_iteration": [round(x, 1) for x in again["step_us"]]}
    del res
    if not a.no_cpu_baseline:
        import oracle
        from oracle import driver_ref

        oracle.load()
        Bs = min(B, 16)
        t0 = time.perf_counter()
        driver_ref.solve(P, xi[:Bs], xr[:Bs], rho[:Bs], N, 2, synth.ALPHAS)
        cw = time.perf_counter() - t0
        rec["cpu_reference"] = {"solve_iterations_per_s": Bs * 2 / cw, "sample": "%d solves x 2 iterations" % Bs,
                                "cores": oracle.num_threads(), "kind": "oracle"}
    print(json.dumps(rec))


# ---------------------------------------------------------------- long-horizon solvers


def solver_sweep(a):
    """gato_direct_solve (block Thomas) and gato_cr_solve (block cyclic reduction) on
    stage-1 outputs of the given configuration's generators, over horizons and batch
    sizes; the batch is 64 generated solves tiled on the device (the solves' times do
    not depend on their values).  Also reports gato_step_solver's choice, which is
    that of the step with its refinement pass: for n <= 16 and N <= 128 it compares the
    refined steps (see --step-sweep), so it can differ there from the faster of these
    two solves alone."""
    import torch

    from block_tridiagonal_pcg_amd import ops, synth

    torch.cuda.set_device(0)

    def timeit(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    rows = []
    for N in (65, 128, 256, 512, 1024):
        base = synth.make_batch(a.config, 64, N=N)
        dev0 = ops.to_device(base)
        n, m = base["dims"][0], base["dims"][1]
        for B in (64, 256, 512, 1024, 2048, 4096):
            if B * N > 2 ** 21:
                continue
            dev = {k: v.repeat(B // 64, *([1] * (v.dim() - 1))).contiguous() for k, v in dev0.items() if k != "dims"}
            dims = (n, m, N, B)
            out = ops.alloc_outputs(dims)
            ops.gato_form_schur(dims, *[dev[f] for f in synth.FIELDS], None, out["S"], out["Pinv"], out["gamma"],
                                out["Qinv"], out["Rinv"], out["flags"])
            args = (out["S"], out["gamma"], out["Qinv"], out["Rinv"], dev["Bu"], dev["q"], dev["r"], out["lam"],
                    out["dz"], out["flags"])
            wd, wc = ops.direct_workspace_for(dims), ops.cr_workspace_for(dims)
            reps = 3 if B * N >= 2 ** 19 else 6
            td = timeit(lambda: ops.gato_direct_solve(dims, *args, wd), reps)
            tc = timeit(lambda: ops.gato_cr_solve(dims, *args, wc), reps)
            choice = ops.gato_step_solver(dims)
            rows.append({"N": N, "B": B, "thomas_us": round(td, 1), "cr_us": round(tc, 1),
                         "faster": "cr" if tc < td else "thomas",
                         "policy": {ops.SOLVER_CR: "cr", ops.SOLVER_THOMAS: "thomas"}.get(choice, "fused")})
            print("N=%4d B=%5d thomas %9.1f us  cr %9.1f us  policy %s" % (N, B, td, tc, rows[-1]["policy"]),
                  file=sys.stderr, flush=True)
            del out, wd, wc, dev
            torch.cuda.empty_cache()
    print(json.dumps({"study": "long-horizon solvers", "workload": synth.CONFIGS[a.config].name,
                      "unit": "us per call", "rows": rows}))


def step_sweep(a):
    """gato_sqp_step_opts with solver CR and with solver THOMAS (refinement on, the step's
    default) on the given configuration's generators over horizons and batch sizes, the
    batch being 64 generated solves tiled on the device; median of 15 calls each, beside
    gato_step_solver's choice for those dims."""
    import numpy as np
    import torch

    from block_tridiagonal_pcg_amd import ops, synth

    torch.cuda.set_device(0)

    def time_step(dims, dev, solver):
        out = ops.alloc_outputs(dims, 8)
        ws = ops.workspace_for(dims, 8, solver=solver)
        call = ops.prepared_sqp_step(dims, *[dev[f] for f in synth.FIELDS], None, 1e-6, 200, synth.ALPHAS, 1.0,
                                     out["lam"], out["dz"], out["merit"], out["merit0"], out["best"], out["iters"],
                                     out["relres"], out["flags"], workspace=ws, solver=solver)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(15):
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    rows = []
    for N in (65, 128, 256, 512):
        base = synth.make_batch(a.config, 64, N=N)
        dev0 = ops.to_device(base)
        n, m = base["dims"][0], base["dims"][1]
        for B in (512, 1024, 1536, 2048, 3072):
            dev = {k: v.repeat((B + 63) // 64, *([1] * (v.dim() - 1)))[:B].contiguous()
                   for k, v in dev0.items() if k != "dims"}
            dims = (n, m, N, B)
            tc = time_step(dims, dev, ops.SOLVER_CR)
            td = time_step(dims, dev, ops.SOLVER_THOMAS)
            choice = ops.gato_step_solver(dims)
            rows.append({"N": N, "B": B, "cr_us": round(tc, 1), "thomas_us": round(td, 1),
                         "faster": "cr" if tc < td else "thomas",
                         "policy": {ops.SOLVER_CR: "cr", ops.SOLVER_THOMAS: "thomas"}.get(choice, "fused")})
            print("N=%4d B=%5d cr %9.1f us  thomas %9.1f us  policy %s" % (N, B, tc, td, rows[-1]["policy"]),
                  file=sys.stderr, flush=True)
            del dev
            torch.cuda.empty_cache()
    print(json.dumps({"study": "long-horizon step, refinement on", "workload": synth.CONFIGS[a.config].name,
                      "unit": "us per step", "rows": rows}))


# ---------------------------------------------------------------- main


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from block_tridiagonal_pcg_amd import ops, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.merit_variants:
        merit_variants(a)
        return
    if a.sqp_driver:
        sqp_driver(a)
        return
    if a.solver_sweep:
        solver_sweep(a)
        return
    if a.step_sweep:
        step_sweep(a)
        return
    torch.cuda.set_device(0)
    refine = a.refine == "on"
    cfg = synth.CONFIGS[a.config]
    batch = synth.make_batch(a.config, a.batch, N=a.horizon)
    batch["cid"] = a.config
    n, m, N, B = batch["dims"]
    n_alpha = 8
    alphas = synth.ALPHAS
    cap = CAPS[a.config]
    dims = batch["dims"]
    dev = ops.to_device(batch)
    out = ops.alloc_outputs(dims, n_alpha)
    ws = ops.workspace_for(dims, n_alpha)
    stream = torch.cuda.current_stream()

    # a plain device copy of 256 MiB: the measured memory rate beside the published peak
    # (and, under the profiler, the reference kernel for scaling its byte counters)
    src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    # pre-marshalled calls (argument checks once, then only the C call per step), each
    # step with its own zeroed starting point
    def prepare(lam):
        return ops.prepared_sqp_step(dims, *[dev[f] for f in synth.FIELDS], None, EPS, cap, alphas, MU, lam,
                                     out["dz"], out["merit"], out["merit0"], out["best"], out["iters"],
                                     out["relres"], out["flags"], workspace=ws, stream=stream,
                                     refine=None if refine else 0)

    warm = prepare(out["lam"])
    for _ in range(a.warmup):
        out["lam"].zero_()
        warm()
    lam0 = torch.zeros((a.steps,) + tuple(out["lam"].shape), dtype=torch.float32, device="cuda")
    steps = [prepare(lam0[k]) for k in range(a.steps)]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for step in steps:
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_avg_s = ev0.elapsed_time(ev1) / 1e3 / a.steps

    # the same K steps again, each between two HIP events on the launch stream (the
    # pages' per-solve statistics: median and 90th percentile of single steps)
    lam0.zero_()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for k, step in enumerate(steps):
        step()
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    per_step_us = np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(a.steps)])
    del evs

    iters = out["iters"].cpu().numpy()
    flags = out["flags"].cpu().numpy()
    if (flags & ~ops.F_LS_FAILED).any():
        print("warning: solves flagged: %s" % np.unique(flags), file=sys.stderr)

    # algorithmic work of one launch (the whole batch)
    solver = ops.gato_step_solver(dims)
    fused = solver == ops.SOLVER_FUSED_PCG
    solve_flops = B * (cr_flops(n, N) if solver == ops.SOLVER_CR else direct_flops(n, m, N))
    flops = B * (form_flops(n, m, N) + recover_flops(n, m, N) + merit_flops(n, m, N, n_alpha)) + \
        (float(iters.sum()) * pcg_iter_flops(n, N) if fused else solve_flops)
    workload = "%s, B=%d" % (cfg.name, B) if a.horizon is None else "%s at N=%d, B=%d" % (cfg.name, N, B)
    traffic = measured_traffic(workload) if fused else None

    # per-stage device times with the three standalone calls (events on the same stream)
    stage_us = ops.stage_times(dims, dev, EPS, cap, alphas, MU, reps=max(3, min(20, a.steps // 10)))
    if fused:
        # one kernel: the timed launches are the dominant kernel
        achieved_tflops = flops / kern_avg_s / 1e12
        kernel, kernel_us = KERNEL, kern_avg_s * 1e6
    else:
        # form, direct solve and merit kernels: the roofline is the solve's, timed like the
        # fused kernel (K back-to-back calls on the step's own stage-1 outputs, HIP events
        # on the launch stream around them)
        kernel = "k_cr_res / k_cr (block cyclic reduction)" if solver == ops.SOLVER_CR else \
            "k_direct (block Thomas)"
        sw = ops.cr_workspace_for(dims) if solver == ops.SOLVER_CR else ops.direct_workspace_for(dims)
        solve = ops.gato_cr_solve if solver == ops.SOLVER_CR else ops.gato_direct_solve
        st1 = ops.alloc_outputs(dims, n_alpha)
        ops.gato_form_schur(dims, *[dev[f] for f in synth.FIELDS], None, st1["S"], st1["Pinv"], st1["gamma"],
                            st1["Qinv"], st1["Rinv"], st1["flags"], stream=stream)
        sargs = (st1["S"], st1["gamma"], st1["Qinv"], st1["Rinv"], dev["Bu"], dev["q"], dev["r"], st1["lam"],
                 st1["dz"], st1["flags"])
        for _ in range(3):
            solve(dims, *sargs, sw, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(a.steps):
            solve(dims, *sargs, sw, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        kernel_us = e0.elapsed_time(e1) * 1e3 / a.steps
        achieved_tflops = solve_flops / (kernel_us * 1e-6) / 1e12
        # the same formed system by PCG (gato_pcg_solve), for its iteration counts: the
        # step itself takes the direct solve at this horizon
        pst = ops.alloc_outputs(dims, n_alpha)
        pcg_us, pcg_iters, pcg_dz = [], None, None
        try:
            for _ in range(3):
                pst["lam"].zero_()
                e0.record(stream)
                ops.gato_pcg_solve(dims, st1["S"], st1["Pinv"], st1["gamma"], st1["Qinv"], st1["Rinv"], dev["A"],
                                   dev["Bu"],
                                   dev["q"], dev["r"], EPS, cap, pst["lam"], pst["dz"], pst["iters"], pst["relres"],
                                   pst["flags"], stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                pcg_us.append(e0.elapsed_time(e1) * 1e3)
        except ops.GatoError as err:
            pcg_alongside = {"note": "gato_pcg_solve does not hold this horizon (%s)" % err}
        else:
            pcg_iters = pst["iters"].cpu().numpy()
            pcg_dz = pst["dz"].cpu().numpy()
            at_cap = (pst["flags"].cpu().numpy() & ops.F_PCG_MAXITER) != 0
            relres = pst["relres"].cpu().numpy()
            pcg_alongside = {
                "note": "stage 2 of the same formed system by gato_pcg_solve (cold start, eps and cap as the "
                        "step's); the step itself takes the direct solve",
                "iters": iters_summary(pcg_iters),
                "at_cap": int(at_cap.sum()),
                "relres_at_cap_max": float(relres[at_cap].max()) if at_cap.any() else None,
                "us_per_call": float(np.median(pcg_us)),
            }
        del st1, sw, pst
    if fused:
        pcg_iters, pcg_alongside, pcg_dz = iters, None, None
    pcg_bytes = float(iters.sum()) * pcg_iter_bytes(n, N)
    pcg_equiv_gbps = pcg_bytes / (stage_us["linsys_us"] * 1e-6) / 1e9 if fused and stage_us["linsys_us"] > 0 else None

    value = B * a.steps / wall
    rec = {
        "metric": "batched SQP-step solves/sec (n=14,m=7,N=64,B=128) + % HBM roofline",
        "value": value,
        "unit": "solves/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": wall / a.steps * 1e3,
        "step_us": {"median": float(np.median(per_step_us)), "p90": float(np.percentile(per_step_us, 90)),
                    "mean": float(per_step_us.mean()), "min": float(per_step_us.min()),
                    "note": "each of K steps between two HIP events on the launch stream, in a second pass"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "n": n, "m": m, "N": N, "B": B, "eps": EPS, "max_iters": cap,
                   "n_alpha": n_alpha, "mu": MU, "lambda0": "zero (cold start: a zeroed buffer per step)",
                   "path": "fused single kernel" if fused else "form + %s%s + merit" % (
                       "block cyclic reduction" if solver == ops.SOLVER_CR else "block Thomas solve",
                       " + one KKT refinement pass" if refine else "")},
        "roofline": {
            "bound": "alu",
            "kernel": kernel,
            "achieved": achieved_tflops,
            "peak": FP32_VECTOR_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved_tflops / FP32_VECTOR_PEAK_TFLOPS,
            "traffic": traffic,
            "flops_per_launch": flops if fused else solve_flops,
            "launch_avg_us": kernel_us,
            "step_launch_avg_us": kern_avg_s * 1e6,
            "copy_GBps": copy_gbps,
            "copy_note": "a 256 MiB device-to-device copy (read + write bytes / time), beside the published "
                         "8 TB/s",
        },
        "pcg_iters": iters_summary(iters),
        "pcg_alongside": pcg_alongside,
        "stage_us_unfused": stage_us,
        "pcg_hbm_equivalent": {
            "algorithmic_bytes": pcg_bytes,
            "achieved_GBps": pcg_equiv_gbps,
            "frac_of_hbm_peak": (pcg_equiv_gbps / HBM_PEAK_GBPS) if pcg_equiv_gbps else None,
            "note": "S and Phi^-1 are register-resident in the PCG kernel; this is the rate the "
                    "same iterations would need from HBM, not HBM traffic",
        },
        "source_sha": source_digest(),
        "pages_context": PAGES_CONTEXT if (n, m, N) == (14, 7, 64) else None,
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"], o_step = cpu_baseline(batch, n_alpha, a.cpu_seconds)
        rec["cpu_baseline"]["gpu_over_cpu"] = value / rec["cpu_baseline"]["value"]
        o_iters = o_step["iters"]
        # the timed step's outputs (every step runs the same cold-started batch) against the
        # oracle's on the whole batch: its PCG step where the step runs PCG, else its exact
        # step (block Cholesky of S, then the recovery and the merits)
        if fused:
            ref, ref_name = o_step, "oracle step (fp64 PCG, same eps and cap)"
        else:
            ref, ref_name = exact_step(batch, n_alpha), "oracle exact step (fp64 block Cholesky of S)"
        dz_err = rel_err_rows(out["dz"].cpu().numpy(), ref["dz"])
        m_err = rel_err_rows(out["merit"].cpu().numpy().reshape(B * n_alpha, 1), ref["merit"].reshape(-1, 1))
        rec["parity_vs_oracle"] = {
            "reference": ref_name, "solves": B, "bar": {"dz_rel": 1e-3, "merit_rel": 1e-4},
            "dz_rel_err": {"median": float(np.median(dz_err)), "max": float(dz_err.max())},
            "merit_rel_err_max": float(m_err.max()),
            "best_equal": int((out["best"].cpu().numpy() == ref["best"]).sum()),
        }
        if pcg_iters is not None:
            # PCG iterations per solve, GPU (fp32) against the oracle (fp64), same solves
            ratio = pcg_iters / np.maximum(o_iters, 1)
            rec["pcg_iters_vs_oracle"] = {
                "gpu": iters_summary(pcg_iters), "oracle": iters_summary(o_iters),
                "gpu_over_oracle": {"min": float(ratio.min()), "median": float(np.median(ratio)),
                                    "max": float(ratio.max())},
                "max_abs_diff": int(np.abs(pcg_iters.astype(np.int64) - o_iters).max())}
            if pcg_dz is not None:
                e = rel_err_rows(pcg_dz, o_step["dz"])
                rec["pcg_iters_vs_oracle"]["pcg_dz_rel_err"] = {"median": float(np.median(e)), "max": float(e.max())}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
