"""Build tests/c_abi/_build/check_mxnorm: a plain-C program that calls the C ABI
of libmxnorm.so (and the CPU oracle, to check it) with no Python involved.
gcc for the host code; the HIP runtime for device memory."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT_DIR = os.path.join(HERE, "_build")
EXE = os.path.join(OUT_DIR, "check_mxnorm")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    lib = os.path.join(ROOT, "mx_quantised_tensor_amd", "lib")
    orc = os.path.join(ROOT, "oracle", "_build")
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(HERE, "check_mxnorm.c"), "-o", tmp,
           "-L", lib, "-lmxnorm", "-L", orc, "-loracle_mx", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../../mx_quantised_tensor_amd/lib:$ORIGIN/../../../oracle/_build"
           ":/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE
