"""Build libgma.so (the HIP library behind include/gma.h) for gfx950, in-tree.

Each .hip translation unit is compiled to an object in parallel, then linked.
Usage:  python -m gaussian_mixture_sequence_gma_amd.build [-j JOBS]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgma.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["gma_api.hip", "gma_bidir.hip", "gma_causal.hip", "gma_proj.hip", "gma_decode.hip",
           "gma_params.hip", "gma_backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 VALU ops stay off: plain fp32 code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # device code assumes finite values (inputs are documented finite):
         # max reductions then fuse with DPP lane moves and need no NaN
         # canonicalisation; host code keeps IEEE NaN semantics
         "-Xarch_device", "-fno-honor-nans",
         "-I" + INCLUDE, "-I" + CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(jobs: int | None = None, only: list | None = None) -> str:
    """Compile every source (or, with `only`, just those, reusing the other
    objects of an earlier build) and link libgma.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    todo = SOURCES if not only else [s for s in SOURCES if s in only]
    # a header newer than any object means every source is rebuilt: the
    # sources share structures through the headers
    objs0 = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    if only and all(os.path.exists(o) for o in objs0):
        oldest = min(os.path.getmtime(o) for o in objs0)
        hdrs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
        hdrs.append(os.path.join(INCLUDE, "gma.h"))
        if any(os.path.getmtime(h) > oldest for h in hdrs):
            todo = SOURCES
    elif only:
        todo = SOURCES
    jobs = jobs or min(len(todo), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized() -> str:
    """libgma_san.so: the library with the host code of gma_api.hip (argument
    checks, planning, workspace sizing, the C ABI) compiled with AddressSanitizer
    and UndefinedBehaviorSanitizer; device code and the other sources as built
    by build().  Load it with clang's ASan runtime preloaded."""
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    for o in objs[1:]:
        if not os.path.exists(o):
            raise RuntimeError("build() first: %s is missing" % o)
    san_obj = os.path.join(OBJDIR, "gma_api_san.o")
    san_flags = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [HIPCC] + FLAGS + san_flags + ["-c", os.path.join(CSRC, SOURCES[0]), "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the sanitized host build:\n" + r.stderr)
    lib = os.path.join(OBJDIR, "libgma_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, san_obj] + objs[1:]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=None)
    ap.add_argument("--only", nargs="*", default=None,
                    help="recompile only these sources (e.g. gma_api.hip)")
    args = ap.parse_args()
    print(build(args.jobs, args.only))
    sys.exit(0)
