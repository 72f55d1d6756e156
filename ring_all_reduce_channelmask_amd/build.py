"""Build the HIP library ``librar.so`` for gfx950 in-tree.

The library holds the ring AllReduce kernel, the host planner and the C ABI
declared in ``include/rar.h``.  Always compiles (the caller decides when).
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "librar.so")
SOURCES = ["csrc/ring_kernel.hip", "csrc/oneshot_kernel.hip", "csrc/plan.cpp", "csrc/capi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep fp32 adds scalar: no packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), "-o", LIB + ".tmp"]
    cmd += ["-x", "hip", *[os.path.join(PKG, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose and res.stderr.strip():
        print("\n".join(l for l in res.stderr.splitlines() if "packed-fp32" not in l))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
