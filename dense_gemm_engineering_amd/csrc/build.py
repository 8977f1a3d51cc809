"""Build the gfx950 GEMM library (libdge_gemm.so) in-tree with hipcc.

Every translation unit is compiled for gfx950 only; the shared library is
written next to the Python package, where the binding loads it.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdge_gemm.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")

SOURCES = ["api.cpp", "kernels_mfma_f16.hip", "kernels_mfma_bf16.hip", "kernels_mfma_f32.hip",
           "kernels_direct_f16.hip", "kernels_direct_bf16.hip",
           "kernels_misc.hip", "kernels_skinny.hip", "kernels_q4.hip",
           "kernels_decode.hip", "kernels_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", HERE,
          "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(HERE, src), "-o", obj] + CFLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, errs))
    return obj, errs


def build(jobs=None, verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))), 16)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, errs in results:
        if errs and verbose:
            print(errs, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
