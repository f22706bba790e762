"""Pins of the oracle's number formats against library routines and the
OCP MX format definitions (CPU only).

* bf16 decode / RNE encode: exhaustive or dense sets, against torch's bf16.
* E4M3 decode: all 256 codes against torch.float8_e4m3fn.
* E4M3 / E2M1 encode: round trip of every code, every midpoint ties to the
  even code, saturation, signed zero, and agreement with numpy's
  round-half-even on a per-binade grid (an independent route).
* E8M0 exponent: every finite bf16 magnitude against exact rational floor(log2).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from tests import npref


def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = npref.bf16_bits_to_f64(bits)
    got = np.array([O.bf16_decode(b) for b in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero
    assert math.copysign(1.0, O.bf16_decode(0x8000)) == -1.0


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(7)
    rnd = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    # every bf16 value, each midpoint between neighbours, and one fp32 ulp either side
    base = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    mids = base | 0x8000
    near = np.concatenate([mids - 1, mids + 1, mids, base])
    near = np.concatenate([near, near | 0x80000000])
    allbits = np.concatenate([rnd, near]).astype(np.uint32)
    f = allbits.view(np.float32)
    got = O.bf16_encode_array(f)
    ref = npref.f32_to_bf16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_bf16_encode_overflow_rounds_to_inf():
    big = np.float32(np.float64(3.3961e38))  # above max bf16 + half ulp
    assert O.bf16_encode_rne(big) == npref.f32_to_bf16_bits(np.array([big]))[0]


def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("elem,ncodes,signbit", [(O.E4M3, 256, 0x80), (O.E2M1, 16, 0x8)])
def test_encode_roundtrip_every_code(elem, ncodes, signbit):
    dec = O.e4m3_decode if elem == O.E4M3 else O.e2m1_decode
    enc = O.e4m3_encode if elem == O.E4M3 else O.e2m1_encode
    for c in range(ncodes):
        v = dec(c)
        if math.isnan(v):
            continue
        assert enc(v) == c, (elem, c, v)
    assert enc(-0.0) == signbit and enc(0.0) == 0


@pytest.mark.parametrize("elem", [O.E4M3, O.E2M1])
def test_midpoints_tie_to_even_code(elem):
    dec = O.e4m3_decode if elem == O.E4M3 else O.e2m1_decode
    enc = O.e4m3_encode if elem == O.E4M3 else O.e2m1_encode
    top = 0x7E if elem == O.E4M3 else 0x7
    for c in range(top):
        lo, hi = dec(c), dec(c + 1)
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert enc(mid) == even, (c, mid)
        assert enc(math.nextafter(mid, -math.inf)) == c
        assert enc(math.nextafter(mid, math.inf)) == c + 1
        # negative side mirrors with the sign bit
        sb = 0x80 if elem == O.E4M3 else 0x8
        assert enc(-mid) == (even | sb)


def test_e4m3_tie_and_saturation_cases():
    assert O.e4m3_encode(432.0) == 0x7E          # 416 | 448 midpoint -> even 448
    assert O.e4m3_encode(2.0 ** -10) == 0x00      # 0 | 2^-9 midpoint -> even 0
    assert O.e4m3_encode(2.0 ** -10 * (1 + 2 ** -20)) == 0x01
    assert O.e4m3_encode(463.99) == 0x7E
    for v in (448.0, 464.0, 479.0, 500.0, 1e30, math.inf):
        assert O.e4m3_encode(v) == 0x7E
        assert O.e4m3_encode(-v) == 0xFE


def test_e2m1_tie_and_saturation_cases():
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             6.0: 7, 6.9: 7, 7.0: 7, 100.0: 7}
    for v, c in cases.items():
        assert O.e2m1_encode(v) == c, v
        assert O.e2m1_encode(-v) == c | 0x8


@pytest.mark.parametrize("elem", [O.E4M3, O.E2M1])
def test_encode_matches_numpy_round_half_even(elem):
    rng = np.random.default_rng(11 + elem)
    vmax = 448.0 if elem == O.E4M3 else 6.0
    # log-uniform magnitudes spanning the subnormal range up past saturation
    mag = np.exp2(rng.uniform(-14, math.log2(vmax) + 1.5, size=300_000))
    v = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32).astype(np.float64)
    codes = O.encode_array(v, elem)  # one unpacked code per value
    dec = O.e4m3_decode if elem == O.E4M3 else O.e2m1_decode
    tab = np.array([dec(c) for c in range(256 if elem == O.E4M3 else 16)])
    got = tab[codes]
    ref = npref.round_elem(v, elem)
    assert np.array_equal(np.abs(got), np.abs(ref))
    sign = (codes >> (7 if elem == O.E4M3 else 3)) & 1
    assert np.array_equal(sign.astype(bool), np.signbit(v))


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-12, math.log2(448.0), size=200_000))
    v = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    # all midpoints between adjacent finite codes, exactly representable in fp32
    pos = np.array([O.e4m3_decode(c) for c in range(127)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.encode_array(v.astype(np.float64), O.E4M3)
    assert np.array_equal(got, ref)


def test_e2m1_value_set_from_grid_definition():
    grid = npref.round_elem(np.linspace(0, 8, 16001), O.E2M1)
    assert sorted(set(grid.tolist())) == sorted(O.e2m1_decode(c) for c in range(8))


def _exact_floor_log2(fr: Fraction) -> int:
    n, d = fr.numerator, fr.denominator
    k = n.bit_length() - d.bit_length()
    # adjust so that 2^k <= n/d < 2^(k+1)
    if Fraction(2) ** k > fr:
        k -= 1
    return k


@pytest.mark.parametrize("emax", [8, 2])
def test_scale_exponent_every_bf16_magnitude(emax):
    for b in range(1, 0x7F80):
        a = O.bf16_decode(b)
        want = max(-127, min(127, _exact_floor_log2(Fraction(a)) - emax))
        assert O.scale_exponent(a, emax) == want, (b, a)
    assert O.scale_exponent(0.0, emax) == -127
    assert O.scale_exponent(math.inf, emax) == 128
    assert O.scale_exponent(math.nan, emax) == 128


@pytest.mark.parametrize("elem", [O.E4M3, O.E2M1])
def test_mx_quant_matches_independent_numpy(elem):
    rng = np.random.default_rng(21 + elem)
    rows, hidden = 64, 512
    x = rng.standard_normal((rows, hidden)).astype(np.float32)
    x *= np.exp2(rng.uniform(-20, 20, size=(rows, 1))).astype(np.float32)
    x[3] = 0.0                                   # an all-zero row
    x[4, :32] = np.float32(1e-39)                # fp32/bf16 subnormal block
    x[5, 64:96] = np.float32(3e38)               # near the top of the range
    x[6, 7] = -0.0
    xb = npref.f32_to_bf16_bits(x)
    codes, scales = O.mx_quant(xb, elem)
    xf = npref.bf16_bits_to_f64(xb)
    q, e = npref.quantise_blocks(xf, elem)
    assert np.array_equal(scales.astype(np.int64), e + 127)
    got = npref.decode_codes(codes, elem, hidden)
    assert np.array_equal(np.abs(got), np.abs(q))
    assert np.array_equal(npref.code_signs(codes, elem, hidden), np.signbit(xf))


def test_mx_quant_nonfinite_block_scale():
    x = np.zeros((1, 64), dtype=np.float32)
    x[0, 5] = np.inf
    x[0, 40] = 1.0
    xb = npref.f32_to_bf16_bits(x)
    xb[0, 50] = 0x7FC1  # a NaN in the second block
    _, scales = O.mx_quant(xb, O.E4M3)
    assert list(scales[0]) == [0xFF, 0xFF]
    x[0, 50] = 2.0
    _, scales = O.mx_quant(npref.f32_to_bf16_bits(x), O.E4M3)
    assert list(scales[0]) == [0xFF, 127 + 1 - 8]


def test_mx_quant_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.mx_quant(np.zeros((2, 48), dtype=np.uint16), O.E4M3)
