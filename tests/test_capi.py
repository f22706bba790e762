"""C ABI of libmxnorm.so on the host (no GPU): the library loads, exports every
function include/mxnorm.h declares, and rejects bad arguments before it
touches the GPU.  Only argument checks run here; no kernel is launched."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import mx_quantised_tensor_amd as mxq
from oracle import derive_c

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxnorm.h")

OK, EINVAL, EALIGN, EUNSUP = 0, -1, -2, -3
A16 = 0x10000    # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10008    # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    L = mxq.lib()
    names = declared_functions()
    assert set(names) >= {"mx_quant", "mxnorm_fwd", "mxnorm_hadamard_fwd", "mxnorm_fwd_ex",
                          "rmsnorm_mxquant_fwd", "mxnorm_bwd", "mxnorm_bwd_workspace_bytes",
                          "mxnorm_default_c", "mxnorm_default_c_for", "mxq_status_str",
                          "mx_quant_gain", "mx_matmul", "mxnorm_linear_fwd"}
    for n in names:
        assert hasattr(L, n), n
    assert mxq.lib().mxq_version().decode().startswith("mxnorm-gfx950")


def test_default_c_matches_derivation():
    for p in (1, 2):
        want = np.float32(derive_c.c_pow2_scale(p))
        assert np.float32(mxq.mxnorm_default_c(p)) == want
        assert np.float32(mxq.lib().mxnorm_default_c(p)) == want
        want = np.float32(derive_c.c_exact_absmax(p))
        assert np.float32(mxq.mxnorm_default_c(p, mxq.SRC_ABSMAX)) == want
    assert mxq.mxnorm_default_c(3) == 0.0
    assert mxq.mxnorm_default_c(2, 2) == 0.0


def _ex(source=0, had=0, **kw):
    a = dict(x=A16, g=None, rows=4, hidden=64, p=2, c=0.0, elem=0, codes=A16, scales=A16,
             rrms=None)
    a.update(kw)
    return mxq.lib().mxnorm_fwd_ex(a["x"], a["g"], a["rows"], a["hidden"], a["p"], a["c"], source,
                                   had, a["elem"], a["codes"], a["scales"], a["rrms"], None)


def test_fwd_ex_argument_checks():
    assert _ex(source=2) == EINVAL
    assert _ex(source=-1) == EINVAL
    assert _ex(source=1, had=8) == EINVAL
    assert _ex(source=1, p=3) == EINVAL
    assert _ex(source=1, hidden=48) == EINVAL
    assert _ex(source=1, x=MIS) == EALIGN
    assert _ex(source=1, rows=0, x=None, codes=None, scales=None) == OK


def test_status_strings():
    for s in (OK, EINVAL, EALIGN, EUNSUP, -4, -5, 7, -2 ** 31, 2 ** 31 - 1):
        assert mxq.status_str(s).startswith("MXQ_")
    assert mxq.status_str(-5) == "MXQ_UNKNOWN"


def test_enum_arguments_outside_their_values_are_rejected():
    # any int is a valid argument value (the enums span int); the checks reject it
    L = mxq.lib()
    for bad in (2, -1, 2 ** 31 - 1, -2 ** 31):
        assert L.mx_quant(A16, 4, 64, bad, A16, A16, None) == EINVAL
        assert L.mxnorm_default_c_for(2, bad) == 0.0
        assert L.mx_matmul(A16, A16, A16, A16, 128, 128, 256, A16, bad, None) == EINVAL


def _mxq(x=A16, rows=4, hidden=64, elem=0, codes=A16, scales=A16):
    return mxq.lib().mx_quant(x, rows, hidden, elem, codes, scales, None)


def _mxn(x=A16, g=None, rows=4, hidden=64, p=2, c=0.0, elem=0, codes=A16, scales=A16, rrms=None):
    return mxq.lib().mxnorm_fwd(x, g, rows, hidden, p, c, elem, codes, scales, rrms, None)


def _had(had=16, **kw):
    a = dict(x=A16, g=None, rows=4, hidden=64, p=2, c=0.0, elem=1, codes=A16, scales=A16,
             rrms=None)
    a.update(kw)
    return mxq.lib().mxnorm_hadamard_fwd(a["x"], a["g"], a["rows"], a["hidden"], a["p"], a["c"],
                                         had, a["elem"], a["codes"], a["scales"], a["rrms"], None)


def _rms(x=A16, g=None, rows=4, hidden=64, eps=1e-5, elem=0, y=A16, codes=A16, scales=A16,
         rstd=None):
    return mxq.lib().rmsnorm_mxquant_fwd(x, g, rows, hidden, eps, elem, y, codes, scales, rstd,
                                         None)


@pytest.mark.parametrize("hidden", [0, -32, 48, 33, 31])
def test_bad_hidden(hidden):
    assert _mxq(hidden=hidden) == EINVAL
    assert _mxn(hidden=hidden) == EINVAL
    assert _had(hidden=hidden) == EINVAL
    assert _rms(hidden=hidden) == EINVAL


def _bwd(x=A16, dy=A16, g=None, rrms=A16, rows=4, hidden=64, dx=A16, dg=None, ws=None):
    return mxq.lib().mxnorm_bwd(x, dy, g, rrms, rows, hidden, dx, dg, ws, None)


def test_hidden_above_limit_unsupported():
    assert _mxq(hidden=mxq.MAX_HIDDEN + 32) == EUNSUP
    assert _mxn(hidden=mxq.MAX_HIDDEN * 2) == EUNSUP
    assert _bwd(hidden=32768 + 32) == EUNSUP


def test_row_count_limit():
    # every launch stays below 2^32 threads: at most 2^24 - 1 rows, 2^34 elements
    assert _mxn(rows=1 << 24) == EUNSUP
    assert _mxq(rows=(1 << 34) // 4096 + 1, hidden=4096) == EUNSUP
    assert _bwd(rows=1 << 24) == EUNSUP


def test_bwd_argument_checks():
    assert _bwd(hidden=48) == EINVAL
    assert _bwd(rows=-1) == EINVAL
    assert _bwd(x=None) == EINVAL
    assert _bwd(rrms=None) == EINVAL
    assert _bwd(dx=None) == EINVAL
    assert _bwd(g=A16) == EINVAL                 # a gain needs dgamma and a workspace
    assert _bwd(g=A16, dg=A16) == EINVAL
    assert _bwd(dy=MIS) == EALIGN
    assert _bwd(dx=MIS) == EALIGN
    assert _bwd(rrms=A16 + 2) == EALIGN
    assert _bwd(g=MIS, dg=A16, ws=A16) == EALIGN
    assert _bwd(g=A16, dg=A16, ws=MIS) == EALIGN
    assert _bwd(rows=0, x=None, dy=None, rrms=None, dx=None) == OK


def test_bwd_workspace_size():
    ws = mxq.mxnorm_bwd_workspace_bytes
    assert ws(0, 4096) == 0
    assert ws(1, 64) == 64 * 4            # one workgroup
    assert ws(5, 64) == 2 * 64 * 4        # ceil(5 / 4) workgroups of 4 waves
    # one wave per row: 512 and 256 workgroups at most for rows of up to 1024
    # and 2048 elements
    assert ws(16384, 2048) == 256 * 2048 * 4
    assert ws(16384, 1024) == 512 * 1024 * 4
    assert ws(16384, 512) == 512 * 512 * 4
    assert ws(1000, 512) == 250 * 512 * 4
    # one row at a time per workgroup of W waves, 512 workgroups at most for
    # W = 2, 3, 5 and 256 for W = 4, 7, 8: rows of 2049..2560 take 5 waves,
    # 2561..3072 3, 3073..3584 7, 3585..4096 8, 4097..4608 2, 4609..8192 8
    assert ws(16384, 2080) == 512 * 2080 * 4      # W = 5, 1 step
    assert ws(16384, 2560) == 512 * 2560 * 4
    assert ws(16384, 2592) == 512 * 2592 * 4      # W = 3, 2 steps
    assert ws(16384, 3072) == 512 * 3072 * 4
    assert ws(16384, 3104) == 256 * 3104 * 4      # W = 7, 1 step
    assert ws(16384, 3584) == 256 * 3584 * 4
    assert ws(16384, 4096) == 256 * 4096 * 4      # W = 8, 1 step
    assert ws(16384, 3616) == 256 * 3616 * 4
    assert ws(16384, 4608) == 512 * 4608 * 4      # W = 2
    assert ws(16384, 4640) == 256 * 4640 * 4      # W = 8, 2 steps
    assert ws(16, 8192) == 16 * 8192 * 4
    assert ws(16384, 8192) == 256 * 8192 * 4
    assert ws(16384, 12288) == 256 * 12288 * 4    # W = 4
    assert ws(16384, 32768) == 256 * 32768 * 4    # W = 8
    assert ws(16, 32800) == 0 and ws(16, 48) == 0 and ws(-1, 64) == 0


def test_negative_rows_and_bad_elem():
    assert _mxq(rows=-1) == EINVAL
    assert _mxn(rows=-5) == EINVAL
    assert _mxq(elem=2) == EINVAL
    assert _mxn(elem=-1) == EINVAL


def test_zero_rows_is_a_noop_even_without_buffers():
    assert _mxq(rows=0, x=None, codes=None, scales=None) == OK
    assert _mxn(rows=0, x=None, codes=None, scales=None) == OK
    assert _had(rows=0, x=None, codes=None, scales=None) == OK
    assert _rms(rows=0, x=None, y=None, codes=None, scales=None) == OK


def test_null_pointers():
    assert _mxq(x=None) == EINVAL
    assert _mxq(codes=None) == EINVAL
    assert _mxn(scales=None) == EINVAL
    assert _rms(y=None) == EINVAL


def test_misaligned_pointers():
    assert _mxq(x=MIS) == EALIGN
    assert _mxq(codes=MIS) == EALIGN
    assert _mxn(g=MIS) == EALIGN
    assert _mxn(rrms=A16 + 2) == EALIGN
    assert _rms(y=MIS) == EALIGN
    assert _rms(rstd=A16 + 1) == EALIGN


@pytest.mark.parametrize("p", [0, 3, -1])
def test_bad_p(p):
    assert _mxn(p=p) == EINVAL
    assert _had(p=p) == EINVAL


@pytest.mark.parametrize("c", [-1.0, math.nan, math.inf])
def test_bad_c(c):
    assert _mxn(c=c) == EINVAL


@pytest.mark.parametrize("had", [0, 8, 64, 17])
def test_bad_had(had):
    assert _had(had=had) == EINVAL


@pytest.mark.parametrize("eps", [-1e-6, math.nan, math.inf])
def test_bad_eps(eps):
    assert _rms(eps=eps) == EINVAL


def test_python_binding_rejects_bad_tensors_on_cpu():
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mxq.mxnorm_fwd(x)          # host tensor
    with pytest.raises(TypeError):
        mxq.mx_quant(torch.zeros((4, 64), dtype=torch.float32))


def _mm(a=A16, as_=A16, b=A16, bs=A16, M=128, N=128, K=256, c=A16, t=0):
    return mxq.lib().mx_matmul(a, as_, b, bs, M, N, K, c, t, None)


def test_matmul_argument_checks():
    assert _mm(K=96) == EUNSUP          # a multiple of 32 but not of 128
    assert _mm(K=131072 + 128) == EUNSUP  # beyond the largest K
    assert _mm(K=100) == EINVAL
    assert _mm(K=0) == EINVAL
    assert _mm(M=-1) == EINVAL
    assert _mm(M=0, a=None, as_=None, c=None) == OK
    assert _mm(a=None) == EINVAL
    assert _mm(a=MIS) == EALIGN
    assert _mm(bs=A16 + 2) == EALIGN
    assert _mm(c=A16 + 2) == EALIGN
    assert _mm(c=A16 + 2, t=1) == EALIGN  # bf16 output: 4-byte aligned too
    assert _mm(t=2) == EINVAL
    assert _mm(t=-1) == EINVAL
    L = mxq.lib()
    assert L.mx_quant_gain(A16, None, 4, 64, 0, A16, A16, None) == EINVAL
    assert L.mx_quant_gain(A16, MIS, 4, 64, 0, A16, A16, None) == EALIGN
    assert L.mxnorm_linear_fwd(A16, 4, 96, 2, 0.0, A16, A16, 8, A16, A16, None, A16, 0,
                               None) == EUNSUP
    assert L.mxnorm_linear_fwd(A16, 4, 128, 2, 0.0, A16, A16, 8, A16, A16, None, A16, 3,
                               None) == EINVAL


def test_linear_fwd_checks_the_product_before_launching():
    # every one of these has a valid activation side: the call must still fail
    # before the norm's launch (on this host a launch would report MXQ_EHIP)
    L = mxq.lib()
    lf = lambda **kw: L.mxnorm_linear_fwd(
        kw.get("x", A16), 4, 128, 2, 0.0, kw.get("wc", A16), kw.get("ws", A16),
        kw.get("n", 8), kw.get("xc", A16), kw.get("xs", A16), None, kw.get("out", A16),
        kw.get("t", 0), None)
    assert lf(wc=None) == EINVAL
    assert lf(ws=None) == EINVAL
    assert lf(out=None) == EINVAL
    assert lf(wc=MIS) == EALIGN
    assert lf(ws=A16 + 2) == EALIGN
    assert lf(xs=A16 + 2) == EALIGN      # the product reads x_scales as dwords
    assert lf(out=A16 + 2) == EALIGN
    assert lf(n=-1) == EINVAL
    assert lf(n=1 << 27) == EUNSUP        # beyond the product's limits
    assert lf(x=None) == EINVAL
    assert lf(n=0, x=None, wc=None, ws=None, out=None) == OK


def test_measure_library_exports_and_checks():
    # the benchmark's byte-pattern references live in their own library, so
    # libmxnorm.so's C ABI holds only calls of the method
    from mx_quantised_tensor_amd import measure
    text = open(os.path.join(ROOT, "include", "mxq_measure.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*int\s+(\w+)\s*\(", text, re.M))
    assert names == {"mxq_pattern_supported", "mxq_measure_pattern", "mxq_bwd_pattern_supported",
                     "mxq_measure_bwd_pattern"}
    M = measure.lib()
    for n in names:
        assert hasattr(M, n), n
    assert not hasattr(mxq.lib(), "mxq_stream_pattern")
    sup = lambda lay, h: M.mxq_pattern_supported(lay, h)
    assert sup(0, 4096) and sup(1, 4096) and sup(2, 4096) and sup(3, 4096) and sup(4, 4096)
    assert sup(0, 512) and not sup(2, 512) and not sup(1, 512) and sup(1, 1024)
    assert not sup(4, 1024) and sup(4, 2048) and not sup(0, 768) and sup(5, 4096)
    assert not sup(5, 1024) and sup(5, 2048) and not sup(6, 4096)
    f = lambda **kw: M.mxq_measure_pattern(kw.get("lay", 0), kw.get("x", A16), kw.get("rows", 4),
                                           kw.get("hidden", 4096), kw.get("codes", A16),
                                           kw.get("scales", A16), kw.get("rrms", A16), None)
    assert f(hidden=768) == EUNSUP
    assert f(lay=7) == EUNSUP
    assert f(hidden=0) == EINVAL
    assert f(rows=-1) == EINVAL
    assert f(rows=0, x=None) == OK
    assert f(x=None) == EINVAL
    assert f(x=MIS) == EALIGN
    assert f(scales=A16 + 2) == EALIGN
    bsup = lambda w, h: M.mxq_bwd_pattern_supported(w, h)
    assert bsup(2, 4096) and bsup(8, 4096) and bsup(2, 1024) and bsup(8, 32768)
    assert not bsup(1, 4096) and not bsup(4, 4096) and not bsup(8, 2048) and not bsup(2, 3072)
    assert not bsup(2, 16384) and not bsup(8, 0)
    bf = lambda **kw: M.mxq_measure_bwd_pattern(kw.get("w", 8), kw.get("x", A16), kw.get("dy", A16),
                                                kw.get("rows", 4), kw.get("hidden", 4096),
                                                kw.get("dx", A16), None)
    assert bf(w=4) == EUNSUP and bf(hidden=3072) == EUNSUP and bf(rows=1 << 24) == EUNSUP
    assert bf(rows=-1) == EINVAL and bf(hidden=0) == EINVAL
    assert bf(rows=0, x=None, dy=None, dx=None) == OK
    assert bf(dy=None) == EINVAL and bf(dx=None) == EINVAL
    assert bf(x=MIS) == EALIGN and bf(dy=A16 + 8) == EALIGN and bf(dx=A16 + 4) == EALIGN


def test_bwd_noalloc_argument_checks_and_scratch_size():
    L = mxq.lib()
    f = lambda **kw: L.mxnorm_bwd_noalloc(
        kw.get("x", A16), kw.get("dy", A16), kw.get("g", A16), kw.get("r", A16),
        kw.get("rows", 4), kw.get("hidden", 256), kw.get("dx", A16), kw.get("dg", A16), None)
    assert f(rows=-1) == EINVAL
    assert f(hidden=48) == EINVAL
    assert f(hidden=32768 + 32) == EUNSUP
    assert f(dg=None) == EINVAL          # a gain needs dgamma
    assert f(x=None) == EINVAL
    assert f(x=MIS) == EALIGN
    assert f(g=MIS) == EALIGN
    assert f(dg=A16 + 2) == EALIGN
    assert f(rows=0, g=None, x=None, dy=None, r=None, dx=None, dg=None) == OK
    # the static scratch covers the workspace of every supported shape
    cap = L.mxnorm_bwd_noalloc_scratch_bytes()
    assert cap == 32 << 20
    need = max(mxq.mxnorm_bwd_workspace_bytes((1 << 24) - 1, h) for h in range(32, 32769, 32))
    assert 0 < need <= cap
