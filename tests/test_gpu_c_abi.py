"""The C ABI from plain C: runs tests/c_abi/_build/check_mxnorm (built by
__graft_entry__.build()), a C program that allocates device memory with the
HIP runtime, calls mx_quant and mxnorm_fwd through include/mxnorm.h and
compares every result with the CPU oracle.  Run with ``pytest -m gpu``."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "_build", "check_mxnorm")


def test_c_program_matches_the_oracle():
    assert os.path.exists(EXE), "build the C check first: python -c 'import __graft_entry__ as g; g.build()'"
    print("case: plain-C check of the C ABI", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c-abi check ok" in r.stdout
    assert r.stdout.count("identical") == 6
