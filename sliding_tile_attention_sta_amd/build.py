"""Build libsta.so (gfx950 HIP kernels + host plan) in-tree.

Usage: python -m sliding_tile_attention_sta_amd.build [--jobs N]

HIP sources are compiled by hipcc for gfx950 only; the host-only plan is
compiled by g++.  Packed fp32 VALU forms are switched off for device code
(``-target-feature -packed-fp32-ops``).  Objects go to ``_build/`` at the
repository root; the shared library lands next to this file.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsta.so")
LIB_DEBUG = os.path.join(PKG, "libsta_debug.so")   # the kernels' bounds checks on (-DSTA_DEBUG)

HIP_SOURCES = ["sta_api.hip", "sta_forward.hip", "sta_backward.hip", "sta_reorder.hip", "sta_search.hip"]
# Per-file extra flags.  The forward kernel needs no IEEE signalling-NaN
# quieting, which lets v_max_f32 read MFMA results without canonicalising them.
# Its instructions are scheduled with the AMDGPU-specific register-pressure
# trackers and without the scheduler's clustered low-occupancy rescheduling
# stage (measured 0.3-0.5 % and a further 0.5-1 % faster on the 720p
# forward, same VGPR count; the backward kernels ran 0.6 % slower with the
# trackers and keep the default).  Loop heads start on 64-byte boundaries, so
# that the key loop's placement does not depend on the size of the code
# before it (unaligned, the same loop measured up to 0.6 % slower).
HIP_EXTRA = {"sta_forward.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee",
                                 "-mllvm", "-amdgpu-use-amdgpu-trackers",
                                 "-mllvm", "-amdgpu-disable-clustered-low-occupancy-reschedule",
                                 "-falign-loops=64"]}
CXX_SOURCES = ["sta_plan.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n  " + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def _plan(debug: bool):
    """Compile commands, objects and output library of one variant."""
    bdir = BUILD + ("_debug" if debug else "")
    os.makedirs(bdir, exist_ok=True)
    extra = ["-DSTA_DEBUG"] if debug else []
    cmds, objs = [], []
    for s in HIP_SOURCES:
        o = os.path.join(bdir, s + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, *HIP_EXTRA.get(s, []), *extra, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in CXX_SOURCES:
        o = os.path.join(bdir, s + ".o")
        cmds.append([CXX, *CXX_FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    return cmds, objs, (LIB_DEBUG if debug else LIB)


def _link(objs, out):
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)


def build_variants(variants=(False, True), jobs: int | None = None, verbose: bool = False) -> list:
    """Compile the given variants (False: libsta.so, True: libsta_debug.so)
    in one pool of compiler processes, the kernel files (the longest
    compiles) first, then link each."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    plans = [_plan(d) for d in variants]
    cmds = [c for cs, _, _ in plans for c in cs]
    slow = ("sta_forward.hip", "sta_backward.hip")
    order = sorted(range(len(cmds)), key=lambda i: 0 if any(x in cmds[i][-3] for x in slow) else 1)
    jobs = jobs or max(1, min(16, os.cpu_count() or 1, len(cmds)))
    with ThreadPoolExecutor(jobs) as ex:
        outs = dict(zip(order, ex.map(_run, [cmds[i] for i in order])))
    if verbose:
        for i, c in enumerate(cmds):
            print(" ".join(c))
            if outs[i].strip():
                print(outs[i])
    for _, objs, out in plans:
        _link(objs, out)
    return [out for _, _, out in plans]


def build(jobs: int | None = None, verbose: bool = False, debug: bool = False) -> str:
    """Compile the library (debug: libsta_debug.so, with -DSTA_DEBUG)."""
    return build_variants((debug,), jobs, verbose)[0]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--debug", action="store_true", help="build libsta_debug.so (kernel bounds checks)")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose, args.debug))


if __name__ == "__main__":
    sys.exit(main())
