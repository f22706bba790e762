"""Build libmxnorm.so (the C ABI + gfx950 HIP kernels) in-tree with hipcc,
and libmxq_measure.so (the benchmark's byte-pattern references).

Output: mx_quantised_tensor_amd/lib/libmxnorm.so and libmxq_measure.so.  Flags:
  * --offload-arch=gfx950: MI355X code objects only;
  * -ffp-contract=off: no implicit FMA, every product and sum rounds once,
    as the method's fp32 steps are defined;
  * -fno-gpu-flush-denormals-to-zero, correctly rounded fp32 / and sqrt;
  * packed fp32 instructions disabled (the compiler would otherwise pair
    independent fp32 multiplies into v_pk_mul_f32).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libmxnorm.so")
SOURCES = ["mxnorm_kernels.hip", "mxnorm_bwd.hip", "mx_gemm.hip", "mxnorm_capi.cpp"]
MEASURE_LIB = os.path.join(LIB_DIR, "libmxq_measure.so")
MEASURE_SOURCES = ["measure.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Build both libraries; returns the path of libmxnorm.so."""
    _link(SOURCES, LIB, verbose)
    _link(MEASURE_SOURCES, MEASURE_LIB, verbose)
    return LIB


def _link(sources, lib, verbose):
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = []
    for src in sources:
        obj = os.path.join(LIB_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
        if verbose and err.strip():
            print(err, flush=True)
        objs.append(obj)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
