"""Builds libveda.so in-tree for gfx950.

    python -m learned_block_sparse_amd.build

Host logic (csrc/host.cpp) is compiled with g++ (no device code, built
without floating-point contraction so its budget arithmetic matches Python's
step for step); the kernels and the C ABI (csrc/*.hip) with hipcc for
gfx950. Objects go to _build/ at the repository root.
"""
from __future__ import annotations

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
LIB = os.path.join(PKG, "libveda.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = [
    "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
    "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    gxx = shutil.which("g++") or "g++"
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for name in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, name)
        obj = os.path.join(BUILD, name + ".o")
        if name.endswith(".hip"):
            jobs.append([hipcc, *HIP_FLAGS, "-c", src, "-o", obj])
        elif name.endswith(".cpp"):
            jobs.append([gxx, *HOST_FLAGS, "-c", src, "-o", obj])
    with ThreadPoolExecutor(max(1, min(8, len(jobs)))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


SANITIZED_HOST_LIB = os.path.join(BUILD, "libveda_host_sanitized.so")


def build_host_sanitized() -> str:
    """The host-only part of libveda (span checks, boxes, budgets, CSR sizing,
    the attend checks: csrc/host.cpp and csrc/api_host.cpp) as its own shared
    library, built with g++ under AddressSanitizer and UndefinedBehavior-
    Sanitizer. It holds no kernel and no launching entry point; tests load it
    with the ASan runtime preloaded to run the host logic under the sanitizers."""
    gxx = shutil.which("g++") or "g++"
    os.makedirs(BUILD, exist_ok=True)
    srcs = [os.path.join(CSRC, n) for n in ("host.cpp", "api_host.cpp")]
    tmp = SANITIZED_HOST_LIB + ".tmp"
    _run([gxx, *HOST_FLAGS, "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared", *srcs,
          "-o", tmp])
    os.replace(tmp, SANITIZED_HOST_LIB)
    return SANITIZED_HOST_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
