"""GPU parity of the MXNormLinear pieces (through the C ABI) against the CPU
oracle: the gain-folded weight cast (bit-exact), the MXFP8 matrix product on
the scaled MFMA instructions (the bar of tests/parity.py, derived from the
matrix unit's measured summation window), and the composed MXNormLinear
forward.  Run on an MI355X with ``pytest -m gpu``."""
import numpy as np
import pytest
import torch

import mx_quantised_tensor_amd as mxq
import oracle as O
from mx_quantised_tensor_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    mxq.lib()
    yield


def rand_mx(rng, rows, K, smin=117, smax=137):
    codes = rng.integers(0, 256, size=(rows, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    scales = rng.integers(smin, smax + 1, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check(ac, as_, bc, bs, what, sample=None, seed=0):
    print("case:", what, flush=True)
    c = mxq.mx_matmul(dev(ac), dev(as_), dev(bc), dev(bs))
    torch.cuda.synchronize()
    c = c.cpu().numpy().astype(np.float64)
    M, N = c.shape
    if sample is None:
        want = O.mx_matmul(ac, as_, bc, bs)
        mn = np.array([(m, n) for m in range(M) for n in range(N)])
        want = want.reshape(-1)
    else:
        rng = np.random.default_rng(seed)
        mn = np.stack([rng.integers(0, M, sample), rng.integers(0, N, sample)], axis=1)
        mn = np.concatenate([mn, [[0, 0], [M - 1, N - 1], [M - 1, 0], [0, N - 1]]])
        want = O.mx_matmul_sampled(ac, as_, bc, bs, mn)
    A, B = P.mx_dequant(ac, as_), P.mx_dequant(bc, bs)
    P.assert_matmul_close(c[mn[:, 0], mn[:, 1]], want, A, B, mn, what)


# K spans 1 .. 16 copy stages of 128, partial scale groups (640, 1152: the
# last group of 4 copy stages is short) and all three rotating scale sets;
# M, N ragged and below, at and above one 256 x 256 tile.
@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 128, 512), (100, 70, 256),
                                   (1, 1, 128), (33, 257, 1024), (130, 384, 2048),
                                   (300, 260, 640), (513, 1000, 1152), (600, 700, 1536)])
def test_matmul_shapes(M, N, K):
    rng = np.random.default_rng(M + 3 * N + K)
    ac, as_ = rand_mx(rng, M, K)
    bc, bs = rand_mx(rng, N, K)
    _check(ac, as_, bc, bs, "M=%d N=%d K=%d" % (M, N, K))


def test_matmul_wide_scale_range_and_nan_scale():
    # scales 2^-47 .. 2^48: every product and sum stays inside the fp32 range
    # (larger ones overflow the fp32 accumulator to Inf, as any fp32 sum would)
    rng = np.random.default_rng(11)
    ac, as_ = rand_mx(rng, 64, 512, 80, 175)
    bc, bs = rand_mx(rng, 96, 512, 80, 175)
    as_[5, 3] = 0xFF
    bs[7, 0] = 0xFF
    _check(ac, as_, bc, bs, "scales 2^-47..2^48 with NaN scales")


def test_matmul_headline_shape_sampled():
    # the 16384 x 4096 activation matrix times a 4096 x 4096 weight
    rng = np.random.default_rng(12)
    ac, as_ = rand_mx(rng, 16384, 4096, 120, 132)
    bc, bs = rand_mx(rng, 4096, 4096, 120, 132)
    _check(ac, as_, bc, bs, "16384x4096x4096 sampled", sample=1500, seed=3)


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (300, 260, 640), (513, 1000, 1152),
                                   (256, 255, 256), (1, 3, 128), (2048, 1024, 512)])
def test_matmul_bf16_output(M, N, K):
    # the bf16 output is the fp32 result rounded to nearest even (torch's
    # float -> bfloat16 cast is RNE): bit-equal to rounding the fp32 output,
    # and within the fp32 bar plus half a bf16 step of the exact product
    rng = np.random.default_rng(M + 5 * N + K)
    ac, as_ = rand_mx(rng, M, K)
    bc, bs = rand_mx(rng, N, K)
    print("case: bf16 out M=%d N=%d K=%d" % (M, N, K), flush=True)
    args = (dev(ac), dev(as_), dev(bc), dev(bs))
    c32 = mxq.mx_matmul(*args)
    c16 = mxq.mx_matmul(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert c16.dtype == torch.bfloat16
    r = c32.to(torch.bfloat16)
    assert torch.equal(c16.view(torch.int16), r.view(torch.int16)), "not RNE of the fp32 result"
    want = O.mx_matmul(ac, as_, bc, bs)
    got = c16.float().cpu().numpy().astype(np.float64)
    mn = np.array([(m, n) for m in range(M) for n in range(N)])
    A, B = P.mx_dequant(ac, as_), P.mx_dequant(bc, bs)
    b32 = P.matmul_bound(A, B, mn)
    bound = b32 + 2.0 ** -8 * (np.abs(want.reshape(-1)) + b32)
    err = np.abs(got.reshape(-1) - want.reshape(-1))
    assert (err <= bound).all(), float((err - bound).max())


def test_matmul_many_tiles_sampled():
    # 17 x 17 = 289 tiles: more tiles than persistent workgroups, and a count
    # that is not a multiple of the 8 XCDs (the round-robin tile order)
    rng = np.random.default_rng(15)
    ac, as_ = rand_mx(rng, 4352, 256, 120, 132)
    bc, bs = rand_mx(rng, 4352, 256, 120, 132)
    _check(ac, as_, bc, bs, "4352x4352x256 sampled", sample=1500, seed=4)


@pytest.mark.parametrize("elem", [0, 1])
def test_quant_gain_exact(elem):
    rng = np.random.default_rng(13 + elem)
    w = W.to_bf16_bits((rng.standard_normal((300, 1024)) * 0.05).astype(np.float32))
    g = W.to_bf16_bits((1 + 0.3 * rng.standard_normal(1024)).astype(np.float32))
    codes, scales = mxq.mx_quant_gain(P.to_device_bf16(w), P.to_device_bf16(g), elem=elem)
    torch.cuda.synchronize()
    oc, os_ = O.mx_quant_gain(w, g, elem)
    P.assert_scales_equal(P.from_device(scales), os_, "quant_gain")
    P.assert_codes(P.from_device(codes), oc, os_, elem, exact=True, what="quant_gain")


def test_mxnorm_linear_forward():
    xb, gb = W.generate(512, 2048, "rowscale", 14)
    rng = np.random.default_rng(14)
    wb = W.to_bf16_bits((rng.standard_normal((384, 2048)) / 45.0).astype(np.float32))
    wc, ws = mxq.mx_quant_gain(P.to_device_bf16(wb), P.to_device_bf16(gb))
    out, xc, xs, rho = mxq.mxnorm_linear_fwd(P.to_device_bf16(xb), wc, ws, p=2)
    torch.cuda.synchronize()
    oxc, oxs, orho = O.mxnorm_fwd(xb, None, 2, mxq.mxnorm_default_c(2), O.E4M3)
    owc, ows = O.mx_quant_gain(wb, gb, O.E4M3)
    assert np.array_equal(P.from_device(xc), oxc) and np.array_equal(P.from_device(xs), oxs)
    assert np.array_equal(P.from_device(rho).view(np.uint32), orho.view(np.uint32))
    assert np.array_equal(P.from_device(wc), owc) and np.array_equal(P.from_device(ws), ows)
    want = O.mx_matmul(oxc, oxs, owc, ows)
    mn = np.array([(m, n) for m in range(0, 512, 3) for n in range(0, 384, 5)])
    A, B = P.mx_dequant(oxc, oxs), P.mx_dequant(owc, ows)
    got = out.cpu().numpy().astype(np.float64)
    P.assert_matmul_close(got[mn[:, 0], mn[:, 1]], want[mn[:, 0], mn[:, 1]], A, B, mn,
                          "mxnorm_linear")
    out16 = mxq.mxnorm_linear_fwd(P.to_device_bf16(xb), wc, ws, p=2, out_dtype=torch.bfloat16)[0]
    torch.cuda.synchronize()
    assert torch.equal(out16.view(torch.int16), out.to(torch.bfloat16).view(torch.int16))
