"""Builds librkv.so (HIP, gfx950) in-tree with hipcc.

The library's build id is a hash of its sources; the Python binding refuses
to load a library whose id does not match the sources next to it, so a stale
build fails loudly instead of being tested.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "librkv.so")
LIB_TIMING_PATH = os.path.join(PKG, "librkv_timing.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # bit-reproducible selection scores: no implicit multiply-add contraction
    "-ffp-contract=off",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))
    return files + [os.path.join(INCLUDE, "rkv.h")]


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sources():
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False, timing: bool = False) -> str:
    """Compile every csrc/*.hip and link librkv.so; returns its path.
    timing=True builds librkv_timing.so instead: the same sources with
    RKV_PHASE_TIMING defined (the fused decode kernel writes per-phase clock
    stamps into rkv_opts.trace), for the phase table only."""
    build_dir = BUILD_DIR + ("_timing" if timing else "")
    os.makedirs(build_dir, exist_ok=True)
    bid = source_hash()
    hipcc = _hipcc()
    flags = HIPCC_FLAGS + [f"-I{INCLUDE}", f"-I{CSRC}", f'-DRKV_BUILD_ID="{bid}"']
    if timing:
        flags.append("-DRKV_PHASE_TIMING")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(build_dir, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [hipcc] + flags + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return r.stderr

    workers = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8")), 16))
    with cf.ThreadPoolExecutor(workers) as ex:
        for warn in ex.map(compile_one, zip(srcs, objs)):
            if verbose and warn:
                print(warn)
    lib_path = LIB_TIMING_PATH if timing else LIB_PATH
    tmp = lib_path + f".tmp{os.getpid()}"
    # --no-undefined: a kernel whose host-side launch stub was not emitted
    # fails here instead of at load time
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    import sys
    print(build(verbose=True, timing="--timing" in sys.argv))
