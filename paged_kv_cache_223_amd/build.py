"""Build libpkv.so in-tree: HIP kernels with hipcc for gfx950, host C++ with g++.

    python paged_kv_cache_223_amd/build.py [--debug]   (a plain script: it must not import the package)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["paged_decode.hip", "decode_vector.hip", "prefill.hip", "kv_append.hip", "copy_blocks.hip", "stream.hip"]
CXX_SOURCES = ["api.cpp", "allocator.cpp"]

# Packed-fp32 instructions are left to nobody: the compiler must not form them.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if verbose and noise:
        print("\n".join(noise))


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source (in parallel, one process per source) and link libpkv.so next to this
    file; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-g"] if debug else []
    steps = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        steps.append((obj, [hipcc, *HIP_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src),
                            "-o", obj]))
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        steps.append((obj, ["g++", *CXX_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src),
                            "-o", obj]))
    workers = max(1, min(len(steps), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for _, cmd in steps]:
            f.result()
    objs = [obj for obj, _ in steps]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp, f"-L{ROCM}/lib", "-lamdhip64"],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, debug="--debug" in sys.argv))
