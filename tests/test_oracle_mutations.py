"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a private copy of the oracle's C source,
builds it, and runs the oracle pin tests against that build; the pins must
fail.  Nothing here touches the GPU path.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mx_oracle.c")

# (name, exact text in mx_oracle.c, replacement) -- first occurrence only
MUTATIONS = [
    ("dropped_sqrt", "float r = (p == 1) ? mu : sqrtf(mu);", "float r = mu;"),
    ("exponent_sign", "return ldexpf(q, 40 / p - E);", "return ldexpf(q, 40 / p + E);"),
    ("dropped_mean", "float mu = Sf / (float)K;", "float mu = Sf;"),
    ("power_ignored", "int t = p * (E - eh);", "int t = (E - eh);"),
    ("ties_away", "return (uint8_t)((lo & 1) ? hi : lo);", "return (uint8_t)hi;"),
    ("e4m3_emax", "return elem == MXO_E4M3 ? 8 : 2;", "return elem == MXO_E4M3 ? 7 : 2;"),
    ("floor_off_by_one", "int e = (k - 1) - emax;", "int e = k - emax;"),
    ("no_low_clamp", "if (e < -127)\n        e = -127;", ""),
    ("gamma_dropped", "yi = yi * (float)mxo_bf16_decode(gamma[col]);\n                y[i] = yi;",
     "y[i] = yi;"),
    ("butterfly_sign", "y[g + j + h] = a - b;", "y[g + j + h] = b - a;"),
    ("nibbles_swapped", "*byte = (uint8_t)((*byte & 0xF0) | c); /* even element: low nibble */",
     "*byte = (uint8_t)((*byte & 0x0F) | (c << 4));"),
    ("bf16_truncates", "pick = (lo & 1) ? hi : lo;", "pick = lo;"),
    ("rms_wrong_count", "ss / (double)hidden", "ss / (double)(hidden - 1)"),
    ("e4m3_subnormal_scale", "mag = ldexp((double)m, -9); /* m/8 * 2^(1-7) */",
     "mag = ldexp((double)m, -10);"),
    # straight-through backward
    ("bwd_no_correction", "dx[r * hidden + j] = rh * gj - corr * mxo_bf16_decode(xr[j]);",
     "dx[r * hidden + j] = rh * gj;"),
    ("bwd_correction_sign", "dx[r * hidden + j] = rh * gj - corr", "dx[r * hidden + j] = rh * gj + corr"),
    ("bwd_rho_squared", "const double corr = rh * rh * rh * dot", "const double corr = rh * rh * dot"),
    ("bwd_divide_by_blocks", "dot / (double)hidden;", "dot / (double)(hidden / 32);"),
    ("bwd_dot_without_gamma", "gk *= mxo_bf16_decode(gamma[k]);", "(void)gk;"),
    ("bwd_dgamma_without_rho", "*\n                       (double)rho[r];", ";"),
    # exact-absmax reading of the block magnitude
    ("absmax_drop_threshold", "if (t <= 24) {\n            uint64_t mp", "if (t <= 20) {\n            uint64_t mp"),
    ("absmax_exponent_offset", "return ldexpf(q, 24 / p + 7 - E);", "return ldexpf(q, 24 / p - E);"),
    ("absmax_power_ignored", "uint64_t mp = (p == 1) ? mk : mk * mk;", "uint64_t mp = mk;"),
    # MXNormLinear pieces
    ("matmul_scale_bias", "return ldexp(mxo_e4m3_decode(codes[k]), (int)s - 127);",
     "return ldexp(mxo_e4m3_decode(codes[k]), (int)s - 128);"),
    ("matmul_block_index", "uint8_t s = scales[k / MXO_BLOCK];", "uint8_t s = scales[k / (2 * MXO_BLOCK)];"),
    ("gain_not_folded", "v[i] = (float)mxo_bf16_decode(w[r * hidden + col]) *\n                       (float)mxo_bf16_decode(gamma[col]);",
     "v[i] = (float)mxo_bf16_decode(w[r * hidden + col]);"),
    ("absmax_no_subnormal_clamp", "if (e < -126)\n        e = -126;\n    *E_k = e;", "*E_k = e;"),
]


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mutated = src.replace(old, new, 1)
    c_path = os.path.join(tmp, name + ".c")
    so_path = os.path.join(tmp, name + ".so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                    "-fopenmp", "-o", so_path, c_path, "-lm"], check=True)
    env = dict(os.environ, MXO_LIB=so_path, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_formats.py", "tests/test_oracle_mxnorm.py",
                        "tests/test_oracle_bwd.py", "tests/test_oracle_absmax.py",
                        "tests/test_oracle_linear.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run_mutant(*m, tmp), MUTATIONS))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, "mutations not caught by the pins: %s" % survivors
