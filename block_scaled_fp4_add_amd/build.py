"""Build liblowbit.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree; nothing is installed.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblowbit.so")
SOURCES = ["gemm_inst_splitk.hip", "gemm_inst_splitk8.hip", "gemm_inst_f80.hip", "gemm_inst_f81.hip",
           "gemm_inst_f82.hip", "gemm_inst_f83.hip", "gemm_inst_nv3.hip", "gemm_inst_mx3.hip", "gemm_inst_nv2.hip", "gemm_inst_nv1.hip", "gemm_inst_nv0.hip", "gemm_inst_mx2.hip",
           "gemm_inst_mx1.hip", "gemm_inst_mx0.hip", "quant.hip", "rope.hip", "sf_layout.hip", "gemm.hip", "api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # packed fp32 math stays off: all fp32 work is scalar or explicit
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, jobs: int = 0) -> str:
    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
        objs.append(obj)
        if len(procs) >= jobs:
            if procs.pop(0).wait() != 0:
                raise RuntimeError("hipcc failed")
    for p in procs:
        if p.wait() != 0:
            raise RuntimeError("hipcc failed")
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
