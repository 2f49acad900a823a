"""Build the HIP library ``libmt.so`` for gfx950 (in-tree).

Each source is compiled to an object in parallel, then linked with hipcc.
HIP sources get ``-Xclang -target-feature -Xclang -packed-fp32-ops`` (no
packed fp32 instructions are generated).  The host source is compiled without
floating-point contraction so that the host Adam rounds exactly once per
operation.

Usage: ``python -m host_memory_centric_amd.build`` (or ``build()``).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmt.so")
ARCH = os.environ.get("MT_OFFLOAD_ARCH", "gfx950")

HIP_SOURCES = ["gemm.hip", "attention.hip", "elementwise.hip", "layer.hip", "prof.hip"]
EXTRA = {}  # per-source extra flags
HOST_SOURCES = ["host.cpp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
          "-Wno-unused-variable"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["-ffp-contract=off", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-pthread"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r.stdout + r.stderr


def build(verbose=False, jobs=None):
    """Compile every source and link libmt.so.  Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([hipcc, *COMMON, *HIP_FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["/opt/rocm/llvm/bin/clang++", *COMMON, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-pthread",
                      "-Wl,-soname,libmt.so"]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                sys.stderr.write(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
