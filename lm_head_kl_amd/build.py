"""Compile the kdkl HIP library for gfx950 in-tree (``lm_head_kl_amd/libkdkl.so``).

Run ``python -m lm_head_kl_amd.build`` (or ``__graft_entry__.build()``).  hipcc
cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "kdkl.hip")
SRC_CACHE = os.path.join(PKG, "csrc", "kdcache.cpp")
OUT = os.path.join(PKG, "libkdkl.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile the library; returns the path of the shared object."""
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           SRC, SRC_CACHE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, OUT)
    build_c_client(verbose)
    return OUT


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi", "kd_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c_abi", "kd_client")


def build_c_client(verbose: bool = False) -> str:
    """Compile the plain-C client of the ABI (tests/c_abi/kd_client) against the
    library just built and the HIP runtime's C API; no HIP device code."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), C_CLIENT_SRC, "-o", C_CLIENT + ".tmp", "-L", PKG, "-lkdkl",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../lm_head_kl_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stdout}")
    os.replace(C_CLIENT + ".tmp", C_CLIENT)
    return C_CLIENT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
