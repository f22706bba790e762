"""GPU parity of the exact-absmax reading of the block magnitude
(mxnorm_fwd_ex with MXQ_SRC_ABSMAX, through the C ABI) against the CPU
oracle on the same seeded inputs.  Run on an MI355X with ``pytest -m gpu``.

Bars as for the E8M0-scale reading: scales byte-equal, rho bit-equal (NaN and
+Inf where the oracle has them), element codes identical."""
import numpy as np
import pytest
import torch

import mx_quantised_tensor_amd as mxq
import oracle as O
from mx_quantised_tensor_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

C_ABS = {1: float.fromhex("0x1.2c6d18p+1"), 2: float.fromhex("0x1.31d9bcp+1")}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    mxq.lib()
    yield


def _check(xb, gb, p, c, elem, had=0, what=""):
    print("case:", what, flush=True)
    x = P.to_device_bf16(xb)
    g = None if gb is None else P.to_device_bf16(gb)
    codes, scales, rho = mxq.mxnorm_fwd_ex(x, g, p=p, c=c, source=mxq.SRC_ABSMAX, had=had,
                                           elem=elem)
    torch.cuda.synchronize()
    oc, os_, orr = O.mxnorm_fwd_ex(xb, gb, p, c, O.SRC_ABSMAX, had, elem)
    gr = P.from_device(rho)
    P.assert_rho_equal(gr, orr, what)
    P.assert_scales_equal(P.from_device(scales), os_, what)
    P.assert_codes(P.from_device(codes), oc, os_, elem, exact=True, what=what)


def _bits(a):
    return W.to_bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("cfg,p", [(1, 2), (2, 1), (2, 2), (3, 2), (4, 2), (5, 2)])
def test_absmax_workloads_full(cfg, p):
    w = W.WORKLOADS[cfg]
    xb, gb = W.workload_inputs(cfg)
    _check(xb, gb, p, C_ABS[p], w.elem, w.had, what=w.name + " absmax")


@pytest.mark.parametrize("hidden", [32, 96, 768, 1056, 2592, 3104, 4096, 4128, 5152, 7168, 8192,
                                    10272, 20480, 32768])
@pytest.mark.parametrize("elem", [0, 1])
def test_absmax_shapes(hidden, elem):
    rows = 37 if hidden <= 8192 else 5
    xb, gb = W.generate(rows, hidden, "rowscale", seed=hidden + 5 * elem)
    for p in (1, 2):
        _check(xb, gb, p, C_ABS[p], elem, what="D=%d p=%d" % (hidden, p))
        _check(xb, None, p, 1.25, elem, what="D=%d p=%d no gamma" % (hidden, p))


@pytest.mark.parametrize("rows", [8192, 8197])
def test_absmax_wave_tail_part(rows):
    # hidden 2048, E4M3, 8192 rows or more: the last 1536 rows are cast by
    # workgroups of one row and 4 waves, with the exact block maxima as well
    xb, gb = W.generate(rows, 2048, "rowscale", seed=rows + 3)
    for p in (1, 2):
        _check(xb, gb, p, C_ABS[p], 0, what="wave tail rows=%d p=%d" % (rows, p))
    _check(xb, None, 2, 1.25, 0, what="wave tail rows=%d no gamma" % rows)


@pytest.mark.parametrize("had", [16, 32])
@pytest.mark.parametrize("hidden", [3072, 4096])
@pytest.mark.parametrize("elem", [0, 1])
def test_absmax_with_rotation(had, hidden, elem):
    xb, gb = W.generate(29, hidden, "outlier", seed=had + hidden + elem)
    _check(xb, gb, 2, C_ABS[2], elem, had=had, what="D=%d H%d absmax" % (hidden, had))
    _check(xb, None, 1, 1.25, elem, had=had, what="D=%d H%d absmax no gamma" % (hidden, had))


def _edge_rows(hidden):
    rng = np.random.default_rng(17)
    base = rng.standard_normal(hidden)
    rows = [np.zeros(hidden), -np.zeros(hidden), base * 1e-39, base * 3e37, base * 1e-30]
    r = base.copy(); r[3] = np.nan; rows.append(r)
    r = base.copy(); r[hidden - 1] = -np.inf; rows.append(r)
    r = np.zeros(hidden); r[0] = 1.0; rows.append(r)
    r = np.zeros(hidden); r[hidden // 2] = 2.0 ** -124; rows.append(r)
    r = np.full(hidden, 1.5 * 2.0 ** 126); rows.append(r)
    r = base * 2.0 ** 100; r[::32] = 3e38; rows.append(r)
    # blocks spread over 2^-60 .. 2^60: terms far below the largest are dropped
    r = base * np.exp2(np.repeat(rng.integers(-60, 60, size=hidden // 32), 32)); rows.append(r)
    # mixed subnormal and normal blocks
    r = base * np.repeat(np.where(np.arange(hidden // 32) % 2 == 0, 1e-39, 1e-37), 32)
    rows.append(r)
    return _bits(np.array(rows))


@pytest.mark.parametrize("elem", [0, 1])
@pytest.mark.parametrize("p", [1, 2])
@pytest.mark.parametrize("hidden", [64, 4096])
def test_absmax_edge_rows(elem, p, hidden):
    xb = _edge_rows(hidden)
    gb = _bits(1 + 0.02 * np.random.default_rng(3).standard_normal(hidden))
    for c in (0.3, 1.0, C_ABS[p], 10.0):
        _check(xb, gb, p, c, elem, what="edge c=%g" % c)
        _check(xb, None, p, c, elem, what="edge no gamma c=%g" % c)


def test_absmax_zero_row_gives_inf_and_nan_scales():
    xb = _bits(np.zeros((2, 256)))
    x = P.to_device_bf16(xb)
    codes, scales, rho = mxq.mxnorm_fwd_ex(x, None, p=2, source=mxq.SRC_ABSMAX)
    torch.cuda.synchronize()
    assert np.isposinf(P.from_device(rho)).all()
    assert (P.from_device(scales) == 0xFF).all()


def test_default_c_used_when_zero():
    xb, gb = W.generate(16, 1024, "outlier", seed=71)
    x, g = P.to_device_bf16(xb), P.to_device_bf16(gb)
    _, _, r0 = mxq.mxnorm_fwd_ex(x, g, p=2, c=0.0, source=mxq.SRC_ABSMAX)
    _, _, r1 = mxq.mxnorm_fwd_ex(x, g, p=2, c=C_ABS[2], source=mxq.SRC_ABSMAX)
    torch.cuda.synchronize()
    assert torch.equal(r0, r1)
