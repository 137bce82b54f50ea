"""Build libdtm_gemm.so in-tree for gfx950 with hipcc.

Every translation unit is compiled separately (in parallel) and linked into
one shared library next to this file.  Device code is built for gfx950 only,
with packed-fp32 instruction selection disabled.

    python -m dense_tiled_matrix_amd.build [-v] [--debug-barriers | --normal-only]

builds both libraries by default (what __graft_entry__.build() runs), so the
debug build never lags the sources; --normal-only builds only
libdtm_gemm.so, --debug-barriers only libdtm_gemm_debug.so (objects in
_build_debug/): the same sources with DTM_DEBUG_BARRIERS=1, which waits for
all outstanding memory operations and adds a workgroup barrier at the top of
every K iteration of the LDS-staged kernels.  Its results must be
bit-identical to the normal library's (an A/B check for missing waits or
barriers); it is slower and meant for tests only.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdtm_gemm.so")
DEBUG_BUILD_DIR = os.path.join(HERE, "_build_debug")
DEBUG_LIB = os.path.join(HERE, "libdtm_gemm_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(DEBUG_BUILD_DIR if debug else BUILD_DIR, os.path.basename(src) + ".o")
    # the .cpp host sources go through hipcc as HIP too (its default for
    # them): give every source the gfx950 device pass, not hipcc's default arch
    cmd = [HIPCC] + COMMON + DEVICE + (["-DDTM_DEBUG_BARRIERS=1"] if debug else [])
    if src.endswith(".hip"):
        cmd += ["-x", "hip"]
    cmd += ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag: harmless
    noise = ("packed-fp32-ops", "not a recognized feature", "unused during compilation")
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def _link(objs, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, jobs: int | None = None, debug_barriers: bool = False) -> str:
    """One of the two libraries: the normal one, or the extra-barrier build."""
    out_dir = DEBUG_BUILD_DIR if debug_barriers else BUILD_DIR
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, os.cpu_count() or 1), 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, debug_barriers), srcs))
    return _link(objs, DEBUG_LIB if debug_barriers else LIB, verbose)


def build_all(verbose: bool = False, jobs: int | None = None) -> tuple[str, str]:
    """Both libraries from one pool of compile jobs (the normal build's
    objects first, so its long compiles start early): libdtm_gemm.so and
    libdtm_gemm_debug.so, kept in step so the debug build always matches the
    sources of the normal one."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(DEBUG_BUILD_DIR, exist_ok=True)
    srcs = sources()
    work = [(s, False) for s in srcs] + [(s, True) for s in srcs]
    jobs = jobs or min(len(work), max(1, os.cpu_count() or 1), 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda w: _compile(w[0], verbose, w[1]), work))
    n = len(srcs)
    return _link(objs[:n], LIB, verbose), _link(objs[n:], DEBUG_LIB, verbose)


if __name__ == "__main__":
    v = "-v" in sys.argv
    if "--normal-only" in sys.argv:
        print(build(verbose=v))
    elif "--debug-barriers" in sys.argv:
        print(build(verbose=v, debug_barriers=True))
    else:
        print("\n".join(build_all(verbose=v)))
