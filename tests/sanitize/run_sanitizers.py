"""Host-side sanitizer run (CPU only, no GPU): builds the CPU oracle and the
host code of libmxnorm.so (argument validation, dispatch) with
AddressSanitizer and UndefinedBehaviorSanitizer, then runs the CPU test suite
(`pytest -m "not gpu"`) against those builds.  The device code of the
library is compiled as usual (sanitizer flags go to the host pass only); the
CPU tests launch no kernel, so what runs instrumented is the oracle and the
C ABI's checks.

    python tests/sanitize/run_sanitizers.py [extra pytest args]

Both libraries use clang's sanitizer runtime (ROCm's clang builds the
oracle here too, so one runtime serves the process), preloaded into Python.
Leak checking is off: the Python interpreter itself holds memory at exit.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "_build")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g"]


def runtime():
    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not found:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return found[0]


def build_oracle():
    lib = os.path.join(OUT, "liboracle_mx_san.so")
    cmd = [CLANG, "-std=c11", "-O1", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra"] + SAN + ["-o", lib, os.path.join(ROOT, "oracle", "mx_oracle.c"),
                                      "-lm"]
    subprocess.run(cmd, check=True)
    return lib


def build_library():
    sys.path.insert(0, ROOT)
    from mx_quantised_tensor_amd import build as B
    lib = os.path.join(OUT, "libmxnorm_san.so")
    host = []
    for f in SAN:  # host pass only: each sanitizer flag behind -Xarch_host
        host += ["-Xarch_host", f]
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + B.FLAGS + host + ["-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
        objs.append(obj)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                    "-fsanitize=address,undefined", "-o", lib] + objs, check=True)
    for o in objs:
        os.remove(o)
    return lib


def main():
    os.makedirs(OUT, exist_ok=True)
    oracle_lib = build_oracle()
    mxq_lib = build_library()
    env = dict(os.environ)
    env.update(MXO_LIB=oracle_lib, MXQ_LIB=mxq_lib, LD_PRELOAD=runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
           "-p", "no:cacheprovider"] + sys.argv[1:]
    print("oracle:", oracle_lib, "\nlibrary:", mxq_lib, "\n" + " ".join(cmd), flush=True)
    sys.exit(subprocess.run(cmd, env=env, cwd=ROOT).returncode)


if __name__ == "__main__":
    main()
