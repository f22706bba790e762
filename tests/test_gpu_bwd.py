"""GPU parity of the straight-through MXNorm backward (libmxnorm.so through
its C ABI) against the fp64 CPU oracle on the same seeded inputs.  Run on an
MI355X with ``pytest -m gpu``.  Bars are in tests/parity.py (dx within one
bf16 ulp plus 2^-16 of its terms; dgamma within 2^-12 of sum |dy x rho|);
dx and dgamma must also be bit-identical from run to run."""
import numpy as np
import pytest
import torch

import mx_quantised_tensor_amd as mxq
import oracle as O
from mx_quantised_tensor_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

C2 = float.fromhex("0x1.c1ed54p+0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    mxq.lib()
    yield


def _inputs(rows, hidden, kind="outlier", seed=21, with_gamma=True):
    xb, gb = W.generate(rows, hidden, kind, seed)
    dyb = W.grad_output(rows, hidden, seed)
    _, _, rho = O.mxnorm_fwd(xb, gb, 2, C2, O.E4M3)
    return xb, dyb, (gb if with_gamma else None), rho


def _run(xb, dyb, gb, rho):
    x, dy = P.to_device_bf16(xb), P.to_device_bf16(dyb)
    g = None if gb is None else P.to_device_bf16(gb)
    r = torch.from_numpy(np.ascontiguousarray(rho)).cuda()
    dx, dg = mxq.mxnorm_bwd(x, dy, r, g)
    torch.cuda.synchronize()
    dxb = P.from_device(dx.view(torch.int16)).view(np.uint16)
    return dxb, (None if dg is None else P.from_device(dg))


def _check(xb, dyb, gb, rho, what):
    print("case:", what, flush=True)
    dxb, dg = _run(xb, dyb, gb, rho)
    ref_dx, ref_dg = O.mxnorm_bwd(xb, dyb, gb, rho)
    P.assert_bwd_close(dxb, dg, xb, dyb, gb, rho, ref_dx, ref_dg, what)
    return dxb, dg


@pytest.mark.parametrize("with_gamma", [True, False])
@pytest.mark.parametrize("hidden", [32, 96, 512, 768, 1024, 1536, 2048, 4064, 4096])
def test_bwd_shapes(hidden, with_gamma):
    for rows in (1, 3, 5, 67):
        xb, dyb, gb, rho = _inputs(rows, hidden, with_gamma=with_gamma, seed=hidden + rows)
        _check(xb, dyb, gb, rho, "rows=%d hidden=%d gamma=%s" % (rows, hidden, with_gamma))


@pytest.mark.parametrize("with_gamma", [True, False])
@pytest.mark.parametrize("hidden", [4128, 6144, 8192, 8224, 10240, 10272, 12288, 14336, 16384,
                                    16416, 20480, 20512, 24576, 28672, 28704, 32768])
def test_bwd_wide_rows(hidden, with_gamma):
    # 2, 4 or 8 waves per row, full and ragged last steps; with a gain, rows
    # above 8192 elements take 5 to 8 steps per wave as the width needs
    # (8224 and 16416: 5 steps with a ragged last one, 10272 and 20512: 6,
    # 14336 and 28672: 7 full ones, 28704: 8)
    for rows in (1, 5, 67):
        xb, dyb, gb, rho = _inputs(rows, hidden, with_gamma=with_gamma, seed=hidden + rows)
        _check(xb, dyb, gb, rho, "rows=%d hidden=%d gamma=%s" % (rows, hidden, with_gamma))


@pytest.mark.parametrize("hidden", [8192, 10240, 16384, 24576, 32768])
def test_bwd_wide_rows_persistent(hidden):
    # more rows than workgroups (512 or 256 of them): each workgroup takes several
    # rows, alternating register sets (W = 2, 4) or one set (W = 8)
    rows = {8192: 1200, 10240: 600, 16384: 600, 24576: 600, 32768: 600}[hidden]
    xb, dyb, gb, rho = _inputs(rows, hidden, kind="rowscale", seed=hidden)
    dx1, dg1 = _check(xb, dyb, gb, rho, "persistent rows=%d hidden=%d" % (rows, hidden))
    dx2, dg2 = _run(xb, dyb, gb, rho)
    assert np.array_equal(dx1, dx2) and np.array_equal(dg1.view(np.uint32), dg2.view(np.uint32))


@pytest.mark.parametrize("with_gamma", [True, False])
@pytest.mark.parametrize("hidden", [2048, 2080, 2336, 2560, 2592, 3072, 3104, 3584, 3616, 3712,
                                    4000, 4096, 4608, 4640, 5120, 7168, 8192])
def test_bwd_multi_wave_bands(hidden, with_gamma):
    # with a gain, rows of 2049..2560 elements take 5 waves of 1 step,
    # 2561..3072 3 waves of 2 steps, 3073..3584 7 waves of 1 step,
    # 3585..4096 8 waves of 1 step and 4609..8192 8 waves of 2 steps, over
    # 256 or 512 persistent workgroups (2048 and 4608: the layouts beside
    # them); without one, rows of 4097..8192 take 8 waves of 2 steps, one row
    # per workgroup; row counts below, at and above the persistent grid,
    # ragged last steps, and the same bits from a second run
    for rows in (1, 255, 257, 700):
        xb, dyb, gb, rho = _inputs(rows, hidden, kind="rowscale", seed=hidden + 7 * rows,
                                   with_gamma=with_gamma)
        dx1, dg1 = _check(xb, dyb, gb, rho, "8-wave band rows=%d hidden=%d" % (rows, hidden))
    dx2, dg2 = _run(xb, dyb, gb, rho)
    assert np.array_equal(dx1, dx2)
    if with_gamma:
        assert np.array_equal(dg1.view(np.uint32), dg2.view(np.uint32))


@pytest.mark.parametrize("kind", ["outlier", "rowscale", "t3"])
def test_bwd_many_rows_persistent(kind):
    # more rows than the persistent grid holds waves: every wave takes several rows
    xb, dyb, gb, rho = _inputs(6000, 1024, kind=kind, seed=31)
    _check(xb, dyb, gb, rho, "6000x1024 " + kind)


def test_bwd_headline_shape_and_reproducible():
    # the 16384 x 4096 activation matrix of the headline forward; dgamma over all
    # rows; dx compared on every row
    xb, _ = W.workload_inputs(3)
    gb = W.workload_inputs(3)[1]
    dyb = W.grad_output(16384, 4096, 3)
    x = P.to_device_bf16(xb)
    g = P.to_device_bf16(gb)
    _, _, rho_d = mxq.mxnorm_fwd(x, g, p=2)
    rho = P.from_device(rho_d)
    dxb, dg = _check(xb, dyb, gb, rho, "16384x4096 rowscale")
    dxb2, dg2 = _run(xb, dyb, gb, rho)
    assert np.array_equal(dxb, dxb2) and np.array_equal(dg.view(np.uint32), dg2.view(np.uint32))


def test_bwd_zero_rows_gives_zero_dgamma():
    g = P.to_device_bf16(W.generate(1, 256, "outlier", 1)[1])
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    r = torch.empty((0,), dtype=torch.float32, device="cuda")
    dg = torch.full((256,), 7.0, dtype=torch.float32, device="cuda")
    dx, dg = mxq.mxnorm_bwd(x, x, r, g, dgamma=dg)
    torch.cuda.synchronize()
    assert dx.shape == (0, 256) and not dg.cpu().numpy().any()


def test_bwd_nonfinite_row_stays_local():
    xb, dyb, gb, rho = _inputs(8, 512, seed=41)
    xb = xb.copy()
    xb[3, 17] = 0x7F80  # +Inf: the forward gives this row rho = NaN
    _, _, rho = O.mxnorm_fwd(xb, gb, 2, C2, O.E4M3)
    assert np.isnan(rho[3])
    dxb, dg = _run(xb, dyb, gb, rho)
    dx = P.bf16_bits_to_f64(dxb)
    assert np.isnan(dx[3]).all()
    keep = np.arange(8) != 3
    ref_dx, _ = O.mxnorm_bwd(xb[keep], dyb[keep], gb, rho[keep])
    P.assert_bwd_close(dxb[keep], None, xb[keep], dyb[keep], gb, rho[keep], ref_dx, None,
                       "finite rows next to a NaN row")
    assert np.isnan(dg).all()  # the NaN row enters every column's sum


def test_bwd_on_side_stream():
    xb, dyb, gb, rho = _inputs(300, 2048, seed=51)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x, dy = P.to_device_bf16(xb), P.to_device_bf16(dyb)
        g = P.to_device_bf16(gb)
        r = torch.from_numpy(rho).cuda()
        dx, dg = mxq.mxnorm_bwd(x, dy, r, g, stream=s)
    s.synchronize()
    ref_dx, ref_dg = O.mxnorm_bwd(xb, dyb, gb, rho)
    P.assert_bwd_close(P.from_device(dx.view(torch.int16)).view(np.uint16), P.from_device(dg),
                       xb, dyb, gb, rho, ref_dx, ref_dg, "side stream")


def test_bwd_maximum_rows_sampled():
    # 2^24 - 1 rows (the C ABI's limit), hidden 64, no gain: dx on sampled rows
    rows, hidden = (1 << 24) - 1, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(32)
    x = torch.randn(rows, hidden, device="cuda", generator=gen).to(torch.bfloat16)
    dy = torch.randn(rows, hidden, device="cuda", generator=gen).to(torch.bfloat16)
    r = (torch.rand(rows, device="cuda", generator=gen) + 0.5).float()
    print("case: mxnorm_bwd rows=%d hidden=%d" % (rows, hidden), flush=True)
    dx, _ = mxq.mxnorm_bwd(x, dy, r, None)
    torch.cuda.synchronize()
    rng = np.random.default_rng(32)
    idx = np.unique(np.concatenate([rng.integers(0, rows, 3000), [0, rows - 1]]))
    ti = torch.from_numpy(idx).cuda()
    xb = x[ti].view(torch.int16).cpu().numpy().view(np.uint16)
    dyb = dy[ti].view(torch.int16).cpu().numpy().view(np.uint16)
    rho = r[ti].cpu().numpy()
    ref_dx, _ = O.mxnorm_bwd(xb, dyb, None, rho)
    got = dx[ti].view(torch.int16).cpu().numpy().view(np.uint16)
    P.assert_bwd_close(got, None, xb, dyb, None, rho, ref_dx, None, "bwd max rows")


@pytest.mark.parametrize("rows", [8191, 8192, 8193, 12289])
@pytest.mark.parametrize("hidden", [2080, 3072, 3584, 4096])
def test_bwd_no_gain_tail_part(rows, hidden):
    # without a gain at 2048 < hidden <= 4096 rows go two per workgroup, and
    # from 8192 rows on the last 4096 one per workgroup of 4 waves: the
    # boundary between the parts, an odd head row count (an empty row slot),
    # ragged widths, and zero / tiny rows placed in the tail part and across
    # the boundary
    xb, gb = W.generate(rows, hidden, "rowscale", rows + hidden)
    xv = P.bf16_bits_to_f64(xb)
    for r in (rows - 1, rows - 4096, rows - 4097):
        if r >= 0:
            xv[r] = 0.0
    xv[rows - 2] *= 2.0 ** -50
    xv[rows - 4098] *= 2.0 ** -120
    xb = W.to_bf16_bits(xv.astype(np.float32))
    dyb = W.grad_output(rows, hidden, rows)
    _, _, rho = O.mxnorm_fwd(xb, gb, 2, C2, O.E4M3)
    dxb, _ = _check(xb, dyb, None, rho, "no-gain tail rows=%d hidden=%d" % (rows, hidden))
    assert np.isfinite(P.bf16_bits_to_f64(dxb)).all()


@pytest.mark.parametrize("rows", [16383, 16384, 16385])
@pytest.mark.parametrize("hidden", [3584, 3616, 4096])
def test_bwd_no_gain_eight_waves_long_launch(rows, hidden):
    # without a gain, launches of 16384 rows or more of 3585..4096 elements
    # take one row per workgroup of 8 waves (16383 rows and 3584 columns:
    # the pairs with their tail part); zero and tiny rows at the end
    xb, _ = W.generate(rows, hidden, "rowscale", rows + 3 * hidden)
    xv = P.bf16_bits_to_f64(xb)
    xv[rows - 1] = 0.0
    xv[rows - 2] *= 2.0 ** -120
    xb = W.to_bf16_bits(xv.astype(np.float32))
    dyb = W.grad_output(rows, hidden, rows + 1)
    _, _, rho = O.mxnorm_fwd(xb, None, 2, C2, O.E4M3)
    dxb, _ = _check(xb, dyb, None, rho, "no-gain long rows=%d hidden=%d" % (rows, hidden))
    assert np.isfinite(P.bf16_bits_to_f64(dxb)).all()


@pytest.mark.parametrize("with_gamma", [True, False])
@pytest.mark.parametrize("hidden", [512, 4096, 8192, 32768])
def test_bwd_zero_and_tiny_rows(hidden, with_gamma):
    # an all-zero row (rho = c 2^119: rho^3 alone overflows fp32), an all -0 row,
    # rows scaled by 2^-50 and 2^-120 (bf16 subnormals), between ordinary rows;
    # every kernel shape: one wave per row, two waves, the wide persistent kernels
    xb, gb = W.generate(6, hidden, "outlier", 61)
    xv = P.bf16_bits_to_f64(xb)
    xv[1] = 0.0
    xv[2] *= 2.0 ** -50
    xv[3] *= 2.0 ** -120
    xb = W.to_bf16_bits(xv.astype(np.float32))
    xb[4] = 0x8000
    dyb = W.grad_output(6, hidden, 61)
    _, _, rho = O.mxnorm_fwd(xb, gb, 2, C2, O.E4M3)
    gb = gb if with_gamma else None
    dxb, dg = _check(xb, dyb, gb, rho, "zero/tiny rows hidden=%d gamma=%s" % (hidden, with_gamma))
    assert np.isfinite(P.bf16_bits_to_f64(dxb)).all()
    if with_gamma:
        assert np.isfinite(dg).all()
