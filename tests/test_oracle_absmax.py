"""Pins of the oracle's exact-absmax reading of the block magnitude (CPU only).

In this reading the power mean runs over the block absmax values themselves
(mt_k = max |x_i| of block k) instead of their power-of-two E8M0 scales.
What fixes the oracle's result (none of it is the oracle checking itself):
  * closed forms -- constant rows give rho = fl(c / |a|); rows of block-constant
    values give 1/RMS (p = 2) or 1/mean|x| (p = 1) with c = 1, checked against
    torch's rms_norm (a library routine) and exact rationals;
  * exact rational sums (fractions) of the power mean with the drop rule on
    tiny random rows, zero and subnormal blocks included;
  * invariants -- 2^j input scaling, block permutation;
  * Theorem 1 of the paper (statistical): with c = E[M^p]^(1/p) (M the max of
    32 |N(0,1)|) the estimate tracks 1/RMS of Gaussian rows;
  * special rows: all-zero (no RMS: +Inf), NaN/Inf (NaN).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from oracle import derive_c
from tests import npref

C_ABS = {1: float(np.float32(derive_c.c_exact_absmax(1))),
         2: float(np.float32(derive_c.c_exact_absmax(2)))}


def bf16(a):
    return npref.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def rho_of(x, p, c, elem=O.E4M3):
    return O.mxnorm_fwd_ex(x, None, p, c, O.SRC_ABSMAX, 0, elem)[2]


@pytest.mark.parametrize("p", [1, 2])
def test_constant_rows(p):
    for a in [1.0, 1.5, -3.0, 0.0078125, 200.0, 2.0 ** 70, -(2.0 ** -90), 3.0 * 2.0 ** -133,
              255.0 * 2.0 ** -120]:
        x = bf16(np.full((1, 256), a))
        av = abs(float(npref.bf16_bits_to_f64(x)[0, 0]))
        for c in (1.0, 1.3125, C_ABS[p]):
            got = rho_of(x, p, c)[0]
            with np.errstate(over="ignore"):
                want = np.float32(c) / np.float32(av)  # one correctly rounded fp32 division
            assert got == want, (a, p, c, got, want)


@pytest.mark.parametrize("p", [1, 2])
def test_block_constant_rows_give_textbook_statistic(p):
    rng = np.random.default_rng(61)
    for trial in range(150):
        K = int(rng.choice([1, 2, 4, 8, 16, 32]))
        # magnitudes within 2^(12/p) of each other: nothing is dropped
        mag = np.exp2(rng.uniform(-10, -10 + 11.5 / p, size=K)) * 2.0 ** rng.integers(-40, 40)
        vals = npref.bf16_bits_to_f64(bf16(mag * rng.choice([-1.0, 1.0], size=K)))
        x = bf16(np.repeat(vals, 32)[None, :])
        got = float(rho_of(x, p, 1.0)[0])
        xr = npref.bf16_bits_to_f64(x)
        if p == 2:
            want = float(torch.rsqrt(torch.mean(torch.tensor(xr) ** 2)))   # rms_norm's rstd, eps 0
            ms = sum(Fraction(float(v)) ** 2 for v in vals) / K
            assert abs(want - 1.0 / math.sqrt(float(ms))) <= 1e-15 * want
        else:
            want = float(K / sum(Fraction(abs(float(v))) for v in vals))
        assert abs(got - want) <= 2.0 ** -21 * want, (trial, got, want)


def _exact_stat(xrow, p):
    """E and the integer S of the reading, by exact rational arithmetic."""
    m = np.abs(npref.bf16_bits_to_f64(xrow)).reshape(-1, 32).max(axis=1)
    Es, Ms = [], []
    for v in m:
        fv = Fraction(float(v))
        if fv == 0:
            Es.append(-126)
            Ms.append(Fraction(0))
            continue
        e = math.floor(math.log2(float(v)))
        while Fraction(2) ** e > fv:
            e -= 1
        while Fraction(2) ** (e + 1) <= fv:
            e += 1
        e = max(e, -126)
        Es.append(e)
        Ms.append(fv / Fraction(2) ** (e - 7))
    E = max(Es)
    S = Fraction(0)
    for e, M in zip(Es, Ms):
        t = p * (E - e)
        if t <= 24:
            S += M ** p * Fraction(2) ** (24 - t)
    assert S.denominator == 1
    return E, int(S)


@pytest.mark.parametrize("p", [1, 2])
def test_power_sum_exact_with_drop_rule(p):
    rng = np.random.default_rng(62)
    for trial in range(300):
        K = int(rng.integers(1, 12))
        base = rng.standard_normal((K, 32)) * np.exp2(rng.integers(-30, 30, size=(K, 1)))
        kind = trial % 5
        if kind == 1:
            base[rng.integers(0, K)] = 0.0                        # a zero block
        elif kind == 2:
            base[rng.integers(0, K)] *= 2.0 ** -140               # a subnormal block
        elif kind == 3:
            base = base * 2.0 ** -128                             # every block subnormal
        x = bf16(base.reshape(1, -1))
        E, S = O.row_stat_absmax(x[0], p)
        Ew, Sw = _exact_stat(x[0], p)
        if Sw == 0:
            assert S == 0
            continue
        assert (E, S) == (Ew, Sw), (trial, E, S, Ew, Sw)


def test_rho_from_stat_steps():
    # rho = fl(c / r) * 2^(24/p + 7 - E), r from fl(fl(S)/K) (and sqrt for p = 2)
    rng = np.random.default_rng(63)
    for _ in range(2000):
        p = int(rng.integers(1, 3))
        K = int(rng.integers(1, 1025))
        S = int(rng.integers(1, 2 ** 49))
        E = int(rng.integers(-100, 100))
        c = float(np.float32(rng.uniform(0.5, 3.0)))
        mu = np.float32(np.float32(S) / np.float32(K))
        r = mu if p == 1 else np.float32(np.sqrt(np.float64(mu)))
        q = np.float32(np.float32(c) / r)
        want = float(np.float32(np.ldexp(np.float64(q), 24 // p + 7 - E)))
        assert O.rho_absmax(E, S, K, p, c) == want


@pytest.mark.parametrize("p", [1, 2])
def test_pow2_scaling_and_permutation(p):
    rng = np.random.default_rng(64)
    x = bf16(rng.standard_normal((8, 1024)) * 3.0)
    r0 = rho_of(x, p, C_ABS[p])
    for j in (-7, 9):
        r1 = rho_of(bf16(npref.bf16_bits_to_f64(x) * 2.0 ** j), p, C_ABS[p])
        assert np.array_equal(r1, (r0.astype(np.float64) * 2.0 ** -j).astype(np.float32))
    perm = rng.permutation(32)
    xp = x.reshape(8, 32, 32)[:, perm, :].reshape(8, 1024)
    assert np.array_equal(rho_of(xp, p, C_ABS[p]), r0)


@pytest.mark.parametrize("p", [1, 2])
def test_theorem1_estimate_tracks_rms(p):
    rng = np.random.default_rng(65)
    x = rng.standard_normal((1024, 4096)) * np.exp2(rng.uniform(-4, 4, size=(1024, 1)))
    xb = bf16(x)
    rho = rho_of(xb, p, C_ABS[p]).astype(np.float64)
    rms = np.sqrt(np.mean(npref.bf16_bits_to_f64(xb) ** 2, axis=1))
    ratio = rho * rms
    assert abs(ratio.mean() - 1.0) < 0.01, ratio.mean()
    assert ratio.std() < 0.03


def test_special_rows():
    z = np.zeros((1, 128), dtype=np.uint16)
    assert rho_of(z, 2, 1.0)[0] == np.inf
    x = bf16(np.ones((2, 128)))
    x[1, 5] = 0x7FC0
    r = rho_of(x, 1, 1.0)
    assert r[0] == 1.0 and np.isnan(r[1])
    _, scales, _ = O.mxnorm_fwd_ex(x, None, 1, 1.0, O.SRC_ABSMAX, 0, O.E4M3)
    assert (scales[1] == 0xFF).all()


def test_scales_source_unchanged_by_the_switch():
    x, g = np.random.default_rng(66).standard_normal((16, 768)), None
    xb = bf16(x)
    a = O.mxnorm_fwd(xb, g, 2, 1.7575276, O.E4M3)
    b = O.mxnorm_fwd_ex(xb, g, 2, 1.7575276, O.SRC_SCALES, 0, O.E4M3)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
