"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_33_amd.build [--jobs N] [--verbose]

Each HIP source compiles to an object under _build/, then one shared library
is linked next to this file.  The build always recompiles: it is the "does it
build" check as much as the build.
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
BUILD = os.path.join(ROOT, "_build", "pagedkv")
LIB = os.path.join(PKG, "libpagedkv.so")

SOURCES = ["api.hip", "cache_write.hip", "decode_valu.hip", "decode_mfma.hip", "multi_mfma.hip",
           "read_tiles.hip",
           "reduce.hip"]
HOST_SOURCES = ["block_manager.cpp", "errors.cpp"]  # host-only C++ (block manager, errors)
ARCH = "gfx950"

# Packed-fp32 instructions are kept out of every kernel: the compiler may not
# form them from plain float code.
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


HOST_CFLAGS = ["-x", "c++", "-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedkv)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that
    # line is expected and not worth showing.
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out)
    return out


def build(jobs: int = 0, verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *HOST_CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(lambda c: _run(c, verbose), cmds):
            pass
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


SANITIZED_LIB = os.path.join(ROOT, "_build", "sanitize", "libpagedkv_host_asan.so")


def build_sanitized(verbose: bool = False) -> str:
    """The host-only part of the library (block manager and error reporting)
    built by g++ with AddressSanitizer and UndefinedBehaviorSanitizer, for CPU
    tests: load it in a process that preloads the ASan runtime."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found")
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    tmp = SANITIZED_LIB + ".tmp"
    _run([gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall",
          "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
          f"-I{INCLUDE}", f"-I{CSRC}",
          *[os.path.join(CSRC, s) for s in HOST_SOURCES], "-o", tmp], verbose)
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(args.jobs, args.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
