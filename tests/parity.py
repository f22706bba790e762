"""Comparison rules between the GPU library and the CPU oracle (tests only).

  * E8M0 scales: byte-equal.
  * rho (rrms): bit-equal, NaN where the oracle has NaN.
  * element codes: the step distance is the difference of ranks in the ordered
    list of representable values (-max ... -0, +0 ... +max); codes under a
    0xFF (NaN) scale are not compared.  The acceptance bar is at most one
    step on at most 0.01% of the elements; the MXNorm kernels are designed to
    reach zero and the tests say which bar they hold.
"""
import numpy as np
import torch


def to_device_bf16(bits: np.ndarray, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def from_device(t):
    return t.detach().cpu().numpy()


def code_ranks(codes: np.ndarray, elem: int) -> np.ndarray:
    """Signed rank of every element code (E2M1 bytes are unpacked)."""
    if elem == 0:
        m = (codes & 0x7F).astype(np.int64)
        neg = (codes & 0x80) != 0
    else:
        lo, hi = codes & 0x0F, codes >> 4
        c = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
        c[..., 0::2] = lo
        c[..., 1::2] = hi
        m = (c & 0x7).astype(np.int64)
        neg = (c & 0x8) != 0
    return np.where(neg, -m - 1, m)


def code_step_stats(got, want, scales_want, elem):
    """(max step, fraction of elements with a nonzero step, count) over the
    elements whose block scale is not NaN."""
    rg, rw = code_ranks(got, elem), code_ranks(want, elem)
    valid = np.repeat(scales_want != 0xFF, 32, axis=-1)
    d = np.abs(rg - rw)[valid]
    if d.size == 0:
        return 0, 0.0, 0
    return int(d.max()), float(np.count_nonzero(d)) / d.size, int(np.count_nonzero(d))


def assert_codes(got, want, scales_want, elem, exact=True, what=""):
    mx, frac, n = code_step_stats(got, want, scales_want, elem)
    if exact:
        assert n == 0, "%s: %d element codes differ (max step %d)" % (what, n, mx)
    else:
        assert mx <= 1 and frac <= 1e-4, "%s: max step %d on %.3g of elements" % (what, mx, frac)


def assert_scales_equal(got, want, what=""):
    bad = np.count_nonzero(got != want)
    assert bad == 0, "%s: %d of %d scales differ" % (what, bad, want.size)


def assert_rho_equal(got, want, what=""):
    gb = got.view(np.uint32)
    wb = want.view(np.uint32)
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), what + ": NaN pattern differs"
    bad = np.count_nonzero(gb[~nan_w] != wb[~nan_w])
    assert bad == 0, "%s: %d of %d rho values differ (max rel %.3g)" % (
        what, bad, want.size,
        np.max(np.abs(got[~nan_w].astype(np.float64) / want[~nan_w] - 1)) if bad else 0)


# ------------------------------------------------------------ straight-through backward
# dx is computed in fp32 as rho (g_j - y_j m), y = fl(rho x), m = fl(sum y g / D),
# and rounded to bf16; the oracle is fp64.  With u = 2^-24 and
# T_j = rho |g_j| + rho^3 |x_j| sum_k |x_k g_k| / D (the sizes of the two terms
# of dx), the fp32 evaluation is within about 80 u T_j of the exact value (the
# rounding of each y, the dot product's FMA chain, tree and wave sums, the
# mean, the FMA and the product by rho); rounding to bf16 adds half a bf16
# ulp.  The bar allows one bf16 ulp of the exact value plus 2^-16 T_j.
# dgamma sums fp32 contributions over rows in chains of at most a few hundred
# additions for the sizes tested: the bar is 2^-12 of sum |dy x rho|.

def bf16_bits_to_f64(bits):
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def assert_bwd_close(dx_bits, dgamma, x_bits, dy_bits, g_bits, rho, ref_dx, ref_dg, what=""):
    x = bf16_bits_to_f64(x_bits)
    gv = bf16_bits_to_f64(dy_bits)
    if g_bits is not None:
        gv = gv * bf16_bits_to_f64(g_bits)[None, :]
    r = rho.astype(np.float64)[:, None]
    d = x.shape[1]
    T = r * np.abs(gv) + r ** 3 * np.abs(x) * np.sum(np.abs(x * gv), axis=1, keepdims=True) / d
    got = bf16_bits_to_f64(dx_bits)
    finite = np.isfinite(ref_dx)
    err = np.abs(got - ref_dx)
    bound = bf16_ulp(ref_dx) + 2.0 ** -16 * T
    bad = finite & ~(err <= bound)
    assert not bad.any(), "%s: dx off at %d elements, worst %r (bound %r)" % (
        what, int(bad.sum()), float(err[bad].max()), float(bound[bad][np.argmax(err[bad])]))
    assert np.array_equal(np.isnan(got), np.isnan(ref_dx)), what + ": NaN pattern of dx"
    if ref_dg is not None:
        scale = np.sum(np.abs(bf16_bits_to_f64(dy_bits) * x * r), axis=0)
        e = np.abs(dgamma.astype(np.float64) - ref_dg)
        ok = e <= 2.0 ** -12 * scale + 1e-30
        assert ok.all(), "%s: dgamma off at %d columns, worst rel %r" % (
            what, int((~ok).sum()), float(np.max(e / np.maximum(scale, 1e-300))))


# ------------------------------------------------------------ MXFP8 matrix product
# The matrix unit sums each 64-element slice of k with a short alignment window
# (probed on gfx950: error up to 2^-11.9 of the slice's largest product, not an
# IEEE sum); slices accumulate in fp32.  Bar per output:
#   2^-10 * sum over slices of max |a_k b_k|  +  (K/64) 2^-23 * sum_k |a_k b_k|.

def e4m3_table():
    import torch
    v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    return v.numpy()


def mx_dequant(codes, scales):
    tab = e4m3_table()
    s = scales.astype(np.float64)
    f = np.where(scales == 0xFF, np.nan, np.exp2(s - 127.0))
    return tab[codes] * np.repeat(f, 32, axis=1)


def matmul_bound(A, B, mn):
    """Error bar for C[m, n] at the listed pairs (A, B dequantised, fp64)."""
    K = A.shape[1]
    out = np.empty(len(mn))
    for t, (m, n) in enumerate(mn):
        p = np.abs(A[m] * B[n]).reshape(K // 64, 64)
        out[t] = 2.0 ** -10 * np.sum(p.max(axis=1)) + (K / 64) * 2.0 ** -23 * np.sum(p)
    return out


def assert_matmul_close(got, want, A, B, mn, what=""):
    bound = matmul_bound(A, B, mn)
    fin = np.isfinite(want)
    assert np.array_equal(np.isnan(got), np.isnan(want)), what + ": NaN pattern"
    err = np.abs(got[fin] - want[fin])
    bad = ~(err <= bound[fin])
    assert not bad.any(), "%s: %d of %d outputs off, worst err %r bound %r" % (
        what, int(bad.sum()), int(fin.sum()), float(err[bad].max()),
        float(bound[fin][bad][np.argmax(err[bad])]))
