"""Ahead-of-time build of the gfx950 attention library (libfa_mi355x.so).

hipcc compiles csrc/fa_fwd.hip (forward) and csrc/fa_bwd.hip (backward) for
gfx950 into a shared library that sits next to this file; the Python binding
loads it with ctypes.  A second library, libfa_mi355x_syncdebug.so, holds the
same kernels built with FA_SYNC_DEBUG for the race check.  Packed-FP32
instruction selection is disabled (-packed-fp32-ops) on purpose.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "fa_fwd.hip"), os.path.join(CSRC, "fa_bwd.hip")]
HEADERS = [os.path.join(CSRC, n) for n in ("fa_sched.h", "exp2_poly.h", "fa_tile.h", "fa_host.h",
                                           "fa_mask_runs.h")] + \
          [os.path.join(ROOT, "include", "fa.h")]
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# The race-check build: the forward and backward kernels compiled with
# FA_SYNC_DEBUG (every wait drains every counter, barriers between the
# pipeline's phases); its results must equal libfa_mi355x.so's bit for bit.
SYNC_DEBUG_LIB_PATH = os.path.join(HERE, "libfa_mi355x_syncdebug.so")
SYNC_DEBUG_SOURCES = list(SOURCES)
TARGETS = [(LIB_PATH, SOURCES, ()),
           (SYNC_DEBUG_LIB_PATH, SYNC_DEBUG_SOURCES, ("FA_SYNC_DEBUG",))]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


COMPILE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                 "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-Wno-inline-asm"]


def hipcc_command(out: str = LIB_PATH):
    """One hipcc line that compiles and links every source (for reference;
    build() runs the same flags per source in parallel, then links)."""
    return [HIPCC] + COMPILE_FLAGS + ["-shared", "-o", out] + SOURCES


def build(out: str = LIB_PATH, verbose: bool = False, defines=(), sources=None) -> str:
    """Compile one library (always recompiles) and return its path; defines
    (e.g. "FA_SYNC_DEBUG") are passed as -D flags."""
    build_many([(out, list(sources or SOURCES), tuple(defines))], verbose)
    return out


def build_all(verbose: bool = False):
    """Compile every library in TARGETS (always recompiles)."""
    build_many(TARGETS, verbose)
    return [t[0] for t in TARGETS]


def build_many(targets, verbose: bool = False):
    """Compile each (output, sources, defines) target: every source of every
    target goes to an object through its own hipcc process, all in
    parallel, then each target is linked."""
    tag = ".tmp%d" % os.getpid()
    jobs = []   # (target index, object, process)
    for ti, (out, sources, defines) in enumerate(targets):
        extra = ["-D" + d for d in defines]
        for src in sources:
            obj = out + "." + os.path.splitext(os.path.basename(src))[0] + tag + ".o"
            cmd = [HIPCC] + COMPILE_FLAGS + extra + ["-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd))
            jobs.append((ti, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                   stderr=subprocess.PIPE, text=True)))
    errs = []
    for _, _, p in jobs:
        _, err = p.communicate()
        if p.returncode != 0:
            errs.append(err[-4000:])
    try:
        if errs:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
        for ti, (out, _, _) in enumerate(targets):
            tmp = out + tag
            objs = [o for t, o, _ in jobs if t == ti]
            cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
            if verbose:
                print(" ".join(cmd))
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc link failed:\n" + r.stderr[-4000:])
            os.replace(tmp, out)
    finally:
        for _, o, _ in jobs:
            if os.path.exists(o):
                os.remove(o)


def is_stale(path: str = LIB_PATH) -> bool:
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build_all(verbose=True))
