"""Build libgato.so in-tree with hipcc for gfx950 (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgato.so")
SOURCES = ["gato.hip", "gato_cr.hip", "gato_driver.hip"]
HEADERS = ["gato_dev.h", "gato_stages.h", "gato_cr.h", "gato_internal.h", "dpp_asm.inc", os.path.join("..", "..", "include", "gato.h"), os.path.join("..", "..", "include", "gato_driver.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(force: bool = True, out: str = LIB, verbose: bool = False) -> str:
    """Generate the DPP blocks and compile the library; returns its path."""
    subprocess.run([sys.executable, os.path.join(CSRC, "gen_dpp_asm.py")], check=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    deps = srcs + [os.path.join(CSRC, h) for h in HEADERS]
    if not force and os.path.exists(out) and all(os.path.getmtime(out) >= os.path.getmtime(d) for d in deps):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objdir = tempfile.mkdtemp(prefix="gato_build_")
    try:
        # each source compiles on its own (they share no device code), side by side
        objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[hipcc()] + HIPCC_FLAGS + inc + ["-c", "-o", o, s] for s, o in zip(srcs, objs)]
        cmds.append([hipcc()] + HIPCC_FLAGS + ["-shared", "-o", tmp] + objs)
        procs = []
        for c in cmds[:-1]:
            if verbose:
                print(" ".join(c), flush=True)
            procs.append(subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        logs = [pr.communicate()[0] for pr in procs]
        for pr, log in zip(procs, logs):
            if pr.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + log)
        if verbose:
            print(" ".join(cmds[-1]), flush=True)
        res = subprocess.run(cmds[-1], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(force=True, verbose=True))
