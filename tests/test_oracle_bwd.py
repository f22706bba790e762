"""Pins of the oracle's straight-through MXNorm backward (CPU only).

The reading pinned here: the MX cast is passed straight through and RMSNorm's
gradient is reused with the forward's rho in place of rstd.  What fixes the
oracle's result (none of it is the oracle checking itself):
  * torch autograd in fp64 of the textbook RMSNorm expression
    y = x * (mean(x^2) + eps)^(-1/2) * gamma, with a per-row eps chosen so that
    its rstd equals the given rho -- RMSNorm's gradient at rstd = rho;
  * torch.nn.functional.rms_norm (a library routine, eps = 0) on rows whose
    MXNorm estimate is exactly 1/RMS (block-constant powers of two, c = 1, p = 2);
  * closed forms and invariants: sum_j x_j dx_j = rho * s * (1 - rho^2 mean(x^2))
    with s = sum_j x_j g_j; gamma = None is gamma = 1; 2^j input scaling.
"""
import numpy as np
import pytest
import torch

import oracle as O
from tests import npref
from mx_quantised_tensor_amd import workloads


def bf16(a):
    return npref.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def f64(bits):
    return npref.bf16_bits_to_f64(bits)


def case(rows, hidden, seed, kind="outlier"):
    """x and gamma from the workload generator, dy ~ N(0, 1), rho from the
    oracle forward (p = 2, default c)."""
    x, g = workloads.generate(rows, hidden, kind, seed)
    dy = workloads.grad_output(rows, hidden, seed)
    _, _, rho = O.mxnorm_fwd(x, g, 2, 1.7575276, O.E4M3)
    return x, dy, g, rho


def term_scale(x, dy, g, rho):
    """Per-element magnitude of the two terms of dx (for relative errors)."""
    xv = f64(x)
    gv = f64(dy) if g is None else f64(dy) * f64(g)[None, :]
    r = rho.astype(np.float64)[:, None]
    d = x.shape[1]
    return r * np.abs(gv) + r ** 3 * np.abs(xv) * np.sum(np.abs(xv * gv), axis=1,
                                                        keepdims=True) / d


def autograd_rmsnorm_at_rho(x, dy, g, rho):
    """RMSNorm's gradient (torch autograd, fp64) at rstd = rho, row by row."""
    xv = torch.tensor(f64(x), requires_grad=True)
    gv = torch.tensor(np.ones(x.shape[1]) if g is None else f64(g), requires_grad=True)
    ms = (xv.detach() ** 2).mean(dim=1, keepdim=True)
    eps = 1.0 / torch.tensor(rho.astype(np.float64))[:, None] ** 2 - ms
    y = xv * torch.rsqrt((xv ** 2).mean(dim=1, keepdim=True) + eps) * gv
    y.backward(torch.tensor(f64(dy)))
    return xv.grad.numpy(), gv.grad.numpy()


@pytest.mark.parametrize("rows,hidden,kind", [(64, 768, "outlier"), (32, 4096, "rowscale"),
                                              (16, 2048, "t3")])
def test_matches_rmsnorm_autograd_at_rstd_rho(rows, hidden, kind):
    x, dy, g, rho = case(rows, hidden, 11, kind)
    dx, dgamma = O.mxnorm_bwd(x, dy, g, rho)
    ref_dx, ref_dg = autograd_rmsnorm_at_rho(x, dy, g, rho)
    err = np.abs(dx - ref_dx) / term_scale(x, dy, g, rho)
    assert err.max() < 1e-12, err.max()
    scale = np.sum(np.abs(f64(dy) * f64(x) * rho.astype(np.float64)[:, None]), axis=0)
    assert np.max(np.abs(dgamma - ref_dg) / scale) < 1e-12


def test_no_gamma_is_unit_gamma():
    x, dy, _, rho = case(32, 1024, 12)
    dx0, dg0 = O.mxnorm_bwd(x, dy, None, rho)
    dx1, _ = O.mxnorm_bwd(x, dy, bf16(np.ones(1024)), rho)
    assert dg0 is None
    assert np.array_equal(dx0, dx1)
    ref_dx, _ = autograd_rmsnorm_at_rho(x, dy, None, rho)
    assert np.max(np.abs(dx0 - ref_dx) / term_scale(x, dy, None, rho)) < 1e-12


def test_library_rms_norm_where_rho_is_one_over_rms():
    rng = np.random.default_rng(13)
    K, rows = 64, 8
    ex = rng.integers(-6, 7, size=(rows, K))
    sg = rng.choice([-1.0, 1.0], size=(rows, K))
    x = bf16(np.repeat(sg * np.exp2(ex.astype(np.float64)), 32, axis=1))
    dy = bf16(rng.standard_normal((rows, K * 32)))
    g = bf16(1.0 + 0.1 * rng.standard_normal(K * 32))
    _, _, rho = O.mxnorm_fwd(x, None, 2, 1.0, O.E4M3)   # = 1/RMS up to fp32 rounding
    dx, dgamma = O.mxnorm_bwd(x, dy, g, rho)
    xt = torch.tensor(f64(x), requires_grad=True)
    gt = torch.tensor(f64(g), requires_grad=True)
    torch.nn.functional.rms_norm(xt, (K * 32,), gt, 0.0).backward(torch.tensor(f64(dy)))
    tol = 2.0 ** -20  # rho is the fp32 rounding of 1/RMS
    assert np.max(np.abs(dx - xt.grad.numpy()) / term_scale(x, dy, g, rho)) < tol
    scale = np.sum(np.abs(f64(dy) * f64(x) * rho.astype(np.float64)[:, None]), axis=0)
    assert np.max(np.abs(dgamma - gt.grad.numpy()) / scale) < tol


def test_projection_closed_form():
    x, dy, g, rho = case(48, 1536, 14)
    dx, _ = O.mxnorm_bwd(x, dy, g, rho)
    xv, gv, r = f64(x), f64(dy) * f64(g)[None, :], rho.astype(np.float64)
    s = np.sum(xv * gv, axis=1)
    ms = np.mean(xv * xv, axis=1)
    lhs = np.sum(xv * dx, axis=1)
    rhs = r * s * (1.0 - r * r * ms)
    bound = 1e-11 * np.sum(np.abs(xv) * term_scale(x, dy, g, rho), axis=1)
    assert np.all(np.abs(lhs - rhs) <= bound)


def test_pow2_scaling_equivariance():
    x, dy, g, rho = case(16, 2048, 15)
    dx, dg = O.mxnorm_bwd(x, dy, g, rho)
    for j in (-3, 5):
        x2 = bf16(f64(x) * 2.0 ** j)
        rho2 = (rho.astype(np.float64) * 2.0 ** -j).astype(np.float32)
        dx2, dg2 = O.mxnorm_bwd(x2, dy, g, rho2)
        assert np.allclose(dx2, dx * 2.0 ** -j, rtol=1e-13, atol=0)
        assert np.allclose(dg2, dg, rtol=1e-13, atol=0)


def test_zero_gradient_and_empty():
    x, dy, g, rho = case(4, 512, 16)
    dx, dg = O.mxnorm_bwd(x, np.zeros_like(dy), g, rho)
    assert not dx.any() and not dg.any()
    dx, dg = O.mxnorm_bwd(x[:0], dy[:0], g, rho[:0])
    assert dx.shape == (0, 512) and not dg.any()


def tiny_rows(hidden, seed):
    """Rows of the outlier generator, then: row 1 all zero (a padding token),
    row 2 scaled by 2^-50, row 3 by 2^-120 (bf16 subnormal and near-subnormal
    values), row 4 all -0."""
    x, g = workloads.generate(6, hidden, "outlier", seed)
    xv = f64(x)
    xv[1] = 0.0
    xv[2] *= 2.0 ** -50
    xv[3] *= 2.0 ** -120
    xb = bf16(xv)
    xb[4] = 0x8000
    dy = workloads.grad_output(6, hidden, seed)
    _, _, rho = O.mxnorm_fwd(xb, g, 2, 1.7575276, O.E4M3)
    return xb, dy, g, rho


@pytest.mark.parametrize("with_gamma", [True, False])
def test_zero_and_tiny_rows(with_gamma):
    # The estimate of an all-zero row is c * 2^(127 - emax) (E4M3: ~1.76 * 2^119);
    # RMSNorm's gradient there is rho * g (the correction term has a zero
    # factor), which is finite; rows of tiny magnitude have a huge rho and
    # still a gradient of ordinary size relative to rho * g.
    x, dy, g, rho = tiny_rows(1024, 17)
    g = g if with_gamma else None
    assert rho[1] == np.float32(1.7575276 * 2.0 ** 119) and rho[4] == rho[1]
    dx, dg = O.mxnorm_bwd(x, dy, g, rho)
    assert np.isfinite(dx).all()
    gv = f64(dy) if g is None else f64(dy) * f64(g)[None, :]
    assert np.array_equal(dx[1], rho[1].astype(np.float64) * gv[1])
    ref_dx, ref_dg = autograd_rmsnorm_at_rho(x, dy, g, rho)
    err = np.abs(dx - ref_dx) / term_scale(x, dy, g, rho)
    assert err.max() < 1e-12, err.max()
    if with_gamma:
        scale = np.sum(np.abs(f64(dy) * f64(x) * rho.astype(np.float64)[:, None]), axis=0)
        assert np.isfinite(dg).all()
        assert np.max(np.abs(dg - ref_dg) / scale) < 1e-12
