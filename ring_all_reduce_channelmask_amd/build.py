"""Build the HIP library ``librar.so`` for gfx950 in-tree.

The library holds the ring AllReduce kernel (one translation unit per payload
type, each instantiating every protocol and reduction operator), the one-shot
kernel, the host planner and the C ABI declared in ``include/rar.h``.  The
sources compile to objects in parallel and are linked once.  Always compiles
(the caller decides when).
"""
import concurrent.futures as cf
import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "librar.so")
SOURCES = ["csrc/ring_kernel_i32.hip", "csrc/ring_kernel_f32.hip", "csrc/ring_kernel_bf16.hip",
           "csrc/oneshot_kernel.hip", "csrc/plan.cpp", "csrc/capi.cpp", "csrc/noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 arithmetic scalar: no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every multiply and add rounds on its own (no fused multiply-add): the
    # results must match the fold the oracle rounds step by step
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res.stderr


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    with tempfile.TemporaryDirectory(prefix="rar_build_") as tmp:
        cmds, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([hipcc, *HIPCC_FLAGS, *inc, "-x", "hip", "-c", os.path.join(PKG, src),
                         "-o", obj])
        with cf.ThreadPoolExecutor(jobs) as pool:
            logs = list(pool.map(_run, cmds))
        link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
        logs.append(_run(link))
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
        for log in logs:
            lines = [l for l in log.splitlines() if "packed-fp32" not in l and l.strip()]
            if lines:
                print("\n".join(lines))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
