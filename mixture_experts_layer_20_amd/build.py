"""Build libmoe.so (HIP, gfx950) in-tree: mixture_experts_layer_20_amd/_lib/libmoe.so.

Usage: python -m mixture_experts_layer_20_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libmoe.so")

SOURCES = ["api.cpp", "route.hip", "router_aux.hip", "dispatch.hip", "combine.hip", "grouped_gemm.hip",
           "grouped_gemm_pipe.hip", "mxfp8.hip"]

ARCH = "gfx950"
# Packed fp32 instructions stay off: plain scalar fp32 code only.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libmoe.so.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libmoe.so failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB_PATH = os.path.join(ASAN_DIR, "libmoe_asan.so")
# Host AddressSanitizer for the C-ABI layer only: the flag applies to the host pass, never to device code.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that a process loading the ASan build must preload."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(llvm)) if os.path.isdir(llvm) else []:
        cand = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise RuntimeError("clang AddressSanitizer runtime not found under " + llvm)


def build_asan(verbose: bool = False) -> str:
    """Debug build: api.cpp (argument checks, workspace layout, scratch set-up) with host ASan,
    linked with the regular objects of the other sources, at _build/asan/libmoe_asan.so."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, s + ".o")) for s in SOURCES):
        build(verbose=verbose)
    os.makedirs(ASAN_DIR, exist_ok=True)
    obj = os.path.join(ASAN_DIR, "api.cpp.o")
    cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, "-O1", "-g", *ASAN_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling api.cpp with ASan failed:\n{r.stderr}")
    objs = [obj] + [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES if s != "api.cpp"]
    r = subprocess.run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", ASAN_LIB_PATH, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking the ASan build failed:\n{r.stderr}")
    if verbose:
        print(ASAN_LIB_PATH)
    return ASAN_LIB_PATH


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--asan", action="store_true", help="also build the host-ASan debug library")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    if a.asan:
        print(build_asan(a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
