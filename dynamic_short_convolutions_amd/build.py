"""Compile the HIP sources under csrc/ into libdsc.so (gfx950), in-tree.

Usage: python -m dynamic_short_convolutions_amd.build [--jobs N] [--incremental]
Cross-compiles without a GPU. Objects go to _build/ at the repository root.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsc.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # packed-fp32 VALU forms stay disabled: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source extra flags. The low-rank forward keeps its MFMA accumulators in
# ordinary VGPRs (no copies out of the accumulation registers), measured faster
# there; the backward kernels hold more accumulators than VGPRs and keep the default.
EXTRA_FLAGS = {
    "lowrank_fwd_w": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = _obj(src)
    extra = [f for prefix, flags in EXTRA_FLAGS.items() if os.path.basename(src).startswith(prefix) for f in flags]
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _obj(src: str) -> str:
    return os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))


def _deps(path: str, seen: set) -> set:
    """The file and every header it reaches through #include "..." (csrc/ and include/)."""
    if path in seen:
        return seen
    seen.add(path)
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#include \""):
                name = line.split('"')[1]
                for d in (os.path.dirname(path), CSRC, INCLUDE):
                    cand = os.path.join(d, name)
                    if os.path.exists(cand):
                        _deps(cand, seen)
                        break
    return seen


def _stale(src: str) -> bool:
    obj = _obj(src)
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in _deps(src, set()))


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every csrc/*.hip and link libdsc.so next to this file. Recompiles everything
    unless `incremental` (then only sources whose file or included headers changed)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not incremental:
        for stale in glob.glob(os.path.join(BUILD, "*.o")):
            os.remove(stale)
    todo = [src for src in srcs if not incremental or _stale(src)]
    jobs = jobs or min(max(len(todo), 1), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, todo))
    objs = [_obj(src) for src in srcs]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources ({len(todo)} compiled)")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--incremental", action="store_true",
                    help="only recompile sources whose file or included headers changed")
    a = ap.parse_args()
    build(a.jobs, verbose=True, incremental=a.incremental)
    sys.exit(0)
