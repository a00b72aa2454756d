"""Builds libkvq.so (the HIP library) in-tree with hipcc for gfx950.

Flags: -ffp-contract=off so fp32 steps stay as written (the encoders are
bit-exact against a fixed operation order; fma appears only where written),
and packed fp32 instructions disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvq.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["kvq_abi.hip", "kvq_encode.hip", "kvq_q4.hip", "kvq_attn.hip", "kvq_sparse.hip", "kvq_q4attn.hip"]
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose=False, jobs=4):
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = ["hipcc", *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), src))
        objs.append(obj)
        if len(procs) >= jobs:
            p, s = procs.pop(0)
            if p.wait() != 0:
                raise RuntimeError(f"hipcc failed on {s}")
    for p, s in procs:
        if p.wait() != 0:
            raise RuntimeError(f"hipcc failed on {s}")
    tmp = LIB + ".tmp"
    _run(["hipcc", "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
