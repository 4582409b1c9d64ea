"""Build libmoe_get.so (the C-ABI HIP library) in-tree for gfx950, its debug
build libmoe_get_debug.so (the same sources with MOE_DEBUG: every layout call
also checks its outputs on the device, see moe_debug_status; loaded by the
binding when MOE_DEBUG=1 is set), and libmoe_ceilings.so, the
bandwidth-ceiling kernels `bench.py --ceilings` times (a separate library:
the product library holds none of them).

    python combine_moe_get_amd/build.py

(run as a script, so that the package -- which loads the library -- is not
imported before the library exists)

Every source is compiled with hipcc for gfx950 only, without fast-math and
with FP contraction off (the combine's FMAs are explicit), and with packed
fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_get.so")
DEBUG_LIB = os.path.join(PKG, "libmoe_get_debug.so")
SOURCES = ["api.hip", "layout.hip", "dispatch.hip", "combine.hip", "quant.hip", "check.hip"]
CEIL_LIB = os.path.join(PKG, "libmoe_ceilings.so")
CEIL_SOURCES = ["ceilings.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
    "-Wno-unused-parameter", "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns about the device-only target feature; drop it
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(job):
        src, debug = job
        stem = os.path.splitext(src)[0] + ("_debug" if debug else "")
        obj = os.path.join(objdir, stem + ".o")
        flags = CFLAGS + (["-DMOE_DEBUG=1"] if debug else [])
        out = _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out:
            print(out, file=sys.stderr)
        return obj

    jobs = [(s, False) for s in SOURCES + CEIL_SOURCES] + [(s, True) for s in SOURCES]
    workers = min(len(jobs), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = dict(zip(jobs, ex.map(compile_one, jobs)))
    for lib, names, debug in ((LIB, SOURCES, False), (DEBUG_LIB, SOURCES, True),
                              (CEIL_LIB, CEIL_SOURCES, False)):
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
              *[objs[(n, debug)] for n in names], "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
