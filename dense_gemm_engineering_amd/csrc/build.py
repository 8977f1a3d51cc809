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
# the diagnostic build: the same library with every pipelined overlap of the
# direct-to-LDS kernels removed by extra waits and barriers
# (GEMM_DIAG_EXTRA_BARRIERS), whose bit-exact results the tests compare with
# the normal build's
LIB_DIAG = os.path.join(PKG, "libdge_gemm_diag.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")

# the longest compiles first, so the parallel build's wall time is the
# longest unit's rather than a long unit started last
SOURCES = ["kernels_direct_f16_nn.hip", "kernels_direct_f16_nt.hip", "kernels_direct_bf16_nn.hip",
           "kernels_direct_bf16_nt.hip", "kernels_q4.hip", "kernels_skinny.hip",
           "kernels_skinny_fold.hip", "kernels_mfma_f16.hip", "kernels_mfma_bf16.hip",
           "kernels_mfma_f32.hip", "kernels_decode.hip", "kernels_misc.hip", "kernels_probe.hip",
           "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", HERE,
          "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


def _compile(job):
    src, diag = job
    obj = os.path.join(OBJDIR + ("_diag" if diag else ""), os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(HERE, src), "-o", obj] + CFLAGS
    if diag:
        cmd.append("-DGEMM_DIAG_EXTRA_BARRIERS=1")
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, errs))
    return obj, errs


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(jobs=None, verbose=False, diag=True):
    """Compile and link libdge_gemm.so (and, with diag, libdge_gemm_diag.so)."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(OBJDIR + "_diag", exist_ok=True)
    work = [(s, d) for s in SOURCES for d in ((False, True) if diag else (False,))]
    jobs = jobs or min(len(work), max(1, len(os.sched_getaffinity(0))), 16)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, work))
    for _, errs in results:
        if errs and verbose:
            print(errs, file=sys.stderr)
    _link([o for (o, _), (_, d) in zip(results, work) if not d], LIB)
    if diag:
        _link([o for (o, _), (_, d) in zip(results, work) if d], LIB_DIAG)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
