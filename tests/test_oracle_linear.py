"""Pins of the oracle's MXNormLinear pieces (CPU only): the gain-folded
weight cast and the MXFP8 x MXFP8 matrix product.

What fixes the oracle's result (none of it is the oracle checking itself):
  * torch's float8_e4m3fn decode (a library routine) with exp2 of the scales
    and numpy's fp64 matmul, an independent evaluation of the same product;
  * exact rational arithmetic (fractions) on tiny shapes;
  * invariants: a shift of every A scale by j multiplies C by 2^j; a NaN
    (0xFF) scale poisons exactly the outputs that use its block;
  * the folded cast against an independent numpy pipeline (per-binade
    rounding) applied to W * gamma, and against the plain cast for gamma = 1;
  * a statistical check that C approximates (x rho)(W gamma)^T within the
    MXFP8 quantisation noise.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from tests import npref
from mx_quantised_tensor_amd import workloads


def rand_mx(rng, rows, K, smin=117, smax=137):
    codes = rng.integers(0, 256, size=(rows, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00          # no NaN codes
    scales = rng.integers(smin, smax + 1, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


def torch_dequant(codes, scales):
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v * np.exp2(np.repeat(scales.astype(np.float64) - 127.0, 32, axis=1))


@pytest.mark.parametrize("M,N,K", [(7, 5, 32), (16, 33, 256), (64, 48, 1024)])
def test_matmul_matches_library_dequant_and_matmul(M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    ac, as_ = rand_mx(rng, M, K)
    bc, bs = rand_mx(rng, N, K)
    c = O.mx_matmul(ac, as_, bc, bs)
    A, B = torch_dequant(ac, as_), torch_dequant(bc, bs)
    ref = A @ B.T
    scale = np.abs(A) @ np.abs(B).T
    assert np.max(np.abs(c - ref) / (scale + 1e-300)) < 1e-14


def test_matmul_exact_fractions_tiny():
    rng = np.random.default_rng(5)
    ac, as_ = rand_mx(rng, 2, 64, 120, 134)
    bc, bs = rand_mx(rng, 3, 64, 120, 134)
    c = O.mx_matmul(ac, as_, bc, bs)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    tab = {c: Fraction(float(v)) for c, v in enumerate(vals.tolist()) if (c & 0x7F) != 0x7F}
    for m in range(2):
        for n in range(3):
            exact = sum(tab[ac[m, k]] * Fraction(2) ** (int(as_[m, k // 32]) - 127) *
                        tab[bc[n, k]] * Fraction(2) ** (int(bs[n, k // 32]) - 127)
                        for k in range(64))
            assert abs(Fraction(c[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + \
                Fraction(1, 2 ** 1000)


def test_scale_shift_and_nan_scale():
    rng = np.random.default_rng(6)
    ac, as_ = rand_mx(rng, 8, 128)
    bc, bs = rand_mx(rng, 6, 128)
    c = O.mx_matmul(ac, as_, bc, bs)
    c3 = O.mx_matmul(ac, (as_.astype(np.int64) + 3).astype(np.uint8), bc, bs)
    assert np.array_equal(c3, c * 8.0)
    bad = as_.copy()
    bad[2, 1] = 0xFF
    cn = O.mx_matmul(ac, bad, bc, bs)
    assert np.isnan(cn[2]).all() and not np.isnan(np.delete(cn, 2, axis=0)).any()


def test_sampled_equals_full():
    rng = np.random.default_rng(7)
    ac, as_ = rand_mx(rng, 20, 256)
    bc, bs = rand_mx(rng, 30, 256)
    c = O.mx_matmul(ac, as_, bc, bs)
    mn = np.stack([rng.integers(0, 20, 50), rng.integers(0, 30, 50)], axis=1)
    s = O.mx_matmul_sampled(ac, as_, bc, bs, mn)
    assert np.array_equal(s, c[mn[:, 0], mn[:, 1]])


def test_quant_gain_matches_numpy_pipeline():
    rng = np.random.default_rng(8)
    w = npref.f32_to_bf16_bits(rng.standard_normal((24, 512)) * 0.05)
    g = npref.f32_to_bf16_bits(1.0 + 0.3 * rng.standard_normal(512))
    codes, scales = O.mx_quant_gain(w, g, O.E4M3)
    prod = (npref.bf16_bits_to_f64(w) * npref.bf16_bits_to_f64(g)[None, :])
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)  # exact in fp32
    q, e = npref.quantise_blocks(prod, O.E4M3)
    assert np.array_equal(scales.astype(np.int64) - 127, e)
    got = npref.decode_codes(codes, O.E4M3, 512)
    assert np.array_equal(got, q)
    c1, s1 = O.mx_quant_gain(w, npref.f32_to_bf16_bits(np.ones(512)), O.E4M3)
    c2, s2 = O.mx_quant(w, O.E4M3)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_mxnorm_linear_approximates_the_unquantised_layer():
    rng = np.random.default_rng(9)
    xb, gb = workloads.generate(64, 1024, "outlier", 9)
    w = npref.f32_to_bf16_bits(rng.standard_normal((96, 1024)) / 32.0)
    xc, xs, rho = O.mxnorm_fwd(xb, None, 2, 1.7575276, O.E4M3)
    wc, ws = O.mx_quant_gain(w, gb, O.E4M3)
    c = O.mx_matmul(xc, xs, wc, ws)
    y = npref.bf16_bits_to_f64(xb) * rho.astype(np.float64)[:, None]
    wg = npref.bf16_bits_to_f64(w) * npref.bf16_bits_to_f64(gb)[None, :]
    ref = y @ wg.T
    rel = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    assert rel < 0.05, rel   # E4M3 carries 3 mantissa bits: ~2^-5 noise per element
