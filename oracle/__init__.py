"""CPU oracle for the MXNorm forward and backward paths -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps the plain C reference in ``mx_oracle.c`` with
numpy arrays; it shares no code with the GPU library and never calls it.

Array conventions: bf16 data travels as ``numpy.uint16`` bit patterns,
row-major ``[rows, hidden]``; codes and scales are ``numpy.uint8``.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

E4M3 = 0
E2M1 = 1
BLOCK = 32
SRC_SCALES = 0   # block magnitude = the E8M0 scale as a power of two
SRC_ABSMAX = 1   # block magnitude = the exact block absmax

_lib = None


def lib():
    """Load the compiled oracle, compiling it first only if it is missing."""
    global _lib
    if _lib is None:
        # MXO_LIB lets the mutation tests load a deliberately broken build.
        path = os.environ.get("MXO_LIB", _build.LIB)
        if not os.path.exists(path):
            _build.build()
        L = C.CDLL(path)
        u16p = C.POINTER(C.c_uint16)
        u8p = C.POINTER(C.c_uint8)
        f32p = C.POINTER(C.c_float)
        i64 = C.c_int64
        L.mxo_bf16_decode.restype = C.c_double
        L.mxo_bf16_decode.argtypes = [C.c_uint16]
        L.mxo_bf16_encode_rne.restype = C.c_uint16
        L.mxo_bf16_encode_rne.argtypes = [C.c_float]
        L.mxo_e4m3_decode.restype = C.c_double
        L.mxo_e4m3_decode.argtypes = [C.c_uint8]
        L.mxo_e2m1_decode.restype = C.c_double
        L.mxo_e2m1_decode.argtypes = [C.c_uint8]
        L.mxo_e4m3_encode.restype = C.c_uint8
        L.mxo_e4m3_encode.argtypes = [C.c_double]
        L.mxo_e2m1_encode.restype = C.c_uint8
        L.mxo_e2m1_encode.argtypes = [C.c_double]
        L.mxo_scale_exponent.restype = C.c_int
        L.mxo_scale_exponent.argtypes = [C.c_double, C.c_int]
        L.mxo_mx_quant.restype = C.c_int
        L.mxo_mx_quant.argtypes = [u16p, i64, i64, C.c_int, u8p, u8p]
        L.mxo_mxnorm_fwd.restype = C.c_int
        L.mxo_mxnorm_fwd.argtypes = [u16p, u16p, i64, i64, C.c_int, C.c_float, C.c_int,
                                     u8p, u8p, f32p]
        L.mxo_mxnorm_hadamard_fwd.restype = C.c_int
        L.mxo_mxnorm_hadamard_fwd.argtypes = [u16p, u16p, i64, i64, C.c_int, C.c_float,
                                              C.c_int, C.c_int, u8p, u8p, f32p]
        L.mxo_rmsnorm_mxquant_fwd.restype = C.c_int
        L.mxo_rmsnorm_mxquant_fwd.argtypes = [u16p, u16p, i64, i64, C.c_float, C.c_int,
                                              u16p, u8p, u8p, f32p]
        L.mxo_row_stat.restype = C.c_int
        L.mxo_row_stat.argtypes = [u16p, i64, C.c_int, C.c_int, C.POINTER(C.c_int),
                                   C.POINTER(C.c_uint64)]
        L.mxo_rho.restype = C.c_float
        L.mxo_rho.argtypes = [C.c_int, C.c_uint64, i64, C.c_int, C.c_float]
        L.mxo_fwht_f32.restype = None
        L.mxo_fwht_f32.argtypes = [f32p, i64, C.c_int]
        L.mxo_bf16_encode_array.restype = None
        L.mxo_bf16_encode_array.argtypes = [f32p, i64, u16p]
        L.mxo_encode_array.restype = None
        L.mxo_encode_array.argtypes = [C.POINTER(C.c_double), i64, C.c_int, u8p]
        L.mxo_max_threads.restype = C.c_int
        L.mxo_max_threads.argtypes = []
        L.mxo_set_threads.restype = None
        L.mxo_set_threads.argtypes = [C.c_int]
        f64p = C.POINTER(C.c_double)
        L.mxo_mx_quant_gain.restype = C.c_int
        L.mxo_mx_quant_gain.argtypes = [u16p, u16p, i64, i64, C.c_int, u8p, u8p]
        L.mxo_mx_dot.restype = C.c_double
        L.mxo_mx_dot.argtypes = [u8p, u8p, u8p, u8p, i64]
        L.mxo_mx_matmul.restype = C.c_int
        L.mxo_mx_matmul.argtypes = [u8p, u8p, u8p, u8p, i64, i64, i64, f64p]
        L.mxo_mx_matmul_sampled.restype = C.c_int
        L.mxo_mx_matmul_sampled.argtypes = [u8p, u8p, u8p, u8p, i64, C.POINTER(C.c_int64), i64,
                                            f64p]
        L.mxo_mxnorm_fwd_ex.restype = C.c_int
        L.mxo_mxnorm_fwd_ex.argtypes = [u16p, u16p, i64, i64, C.c_int, C.c_float, C.c_int,
                                        C.c_int, C.c_int, u8p, u8p, f32p]
        L.mxo_row_stat_absmax.restype = C.c_int
        L.mxo_row_stat_absmax.argtypes = [u16p, i64, C.c_int, C.POINTER(C.c_int),
                                          C.POINTER(C.c_uint64)]
        L.mxo_rho_absmax.restype = C.c_float
        L.mxo_rho_absmax.argtypes = [C.c_int, C.c_uint64, i64, C.c_int, C.c_float]
        L.mxo_mxnorm_bwd.restype = C.c_int
        L.mxo_mxnorm_bwd.argtypes = [u16p, u16p, u16p, f32p, i64, i64, f64p, f64p]
        _lib = L
    return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.POINTER(ctype))


def _bf16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 data must be passed as uint16 bit patterns")
    return a


def emax(elem):
    return 8 if elem == E4M3 else 2


def codes_cols(hidden, elem):
    return hidden if elem == E4M3 else hidden // 2


def _check(status, name):
    if status != 0:
        raise ValueError("%s: invalid arguments (status %d)" % (name, status))


# ---- scalar / bulk format helpers -------------------------------------------------

def bf16_decode(b):
    return lib().mxo_bf16_decode(int(b))


def bf16_encode_rne(f):
    return lib().mxo_bf16_encode_rne(float(f))


def bf16_encode_array(f32):
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    out = np.empty(f32.shape, dtype=np.uint16)
    lib().mxo_bf16_encode_array(_ptr(f32, C.c_float), f32.size, _ptr(out, C.c_uint16))
    return out


def e4m3_decode(c):
    return lib().mxo_e4m3_decode(int(c))


def e2m1_decode(c):
    return lib().mxo_e2m1_decode(int(c))


def e4m3_encode(v):
    return lib().mxo_e4m3_encode(float(v))


def e2m1_encode(v):
    return lib().mxo_e2m1_encode(float(v))


def encode_array(v, elem):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().mxo_encode_array(_ptr(v, C.c_double), v.size, elem, _ptr(out, C.c_uint8))
    return out


def scale_exponent(amax, em):
    return lib().mxo_scale_exponent(float(amax), int(em))


def row_stat(xrow, p, elem):
    xrow = _bf16(xrow)
    E = C.c_int()
    S = C.c_uint64()
    _check(lib().mxo_row_stat(_ptr(xrow, C.c_uint16), xrow.size, p, emax(elem),
                              C.byref(E), C.byref(S)), "row_stat")
    return E.value, S.value


def rho(E, S, K, p, c):
    return lib().mxo_rho(int(E), int(S), int(K), int(p), float(c))


def fwht_f32(y, had):
    y = np.array(y, dtype=np.float32, copy=True)
    lib().mxo_fwht_f32(_ptr(y, C.c_float), y.size, had)
    return y


# ---- whole-matrix entry points (same names as the GPU library) --------------------

def mx_quant(x, elem):
    x = _bf16(x)
    rows, hidden = x.shape
    codes = np.zeros((rows, codes_cols(hidden, elem)), dtype=np.uint8)
    scales = np.zeros((rows, hidden // BLOCK), dtype=np.uint8)
    _check(lib().mxo_mx_quant(_ptr(x, C.c_uint16), rows, hidden, elem,
                              _ptr(codes, C.c_uint8), _ptr(scales, C.c_uint8)), "mx_quant")
    return codes, scales


def mxnorm_fwd(x, gamma, p, c, elem):
    x = _bf16(x)
    rows, hidden = x.shape
    g = None if gamma is None else _bf16(gamma)
    codes = np.zeros((rows, codes_cols(hidden, elem)), dtype=np.uint8)
    scales = np.zeros((rows, hidden // BLOCK), dtype=np.uint8)
    rrms = np.zeros((rows,), dtype=np.float32)
    _check(lib().mxo_mxnorm_fwd(_ptr(x, C.c_uint16), _ptr(g, C.c_uint16), rows, hidden,
                                p, c, elem, _ptr(codes, C.c_uint8), _ptr(scales, C.c_uint8),
                                _ptr(rrms, C.c_float)), "mxnorm_fwd")
    return codes, scales, rrms


def mxnorm_hadamard_fwd(x, gamma, p, c, had, elem):
    x = _bf16(x)
    rows, hidden = x.shape
    g = None if gamma is None else _bf16(gamma)
    codes = np.zeros((rows, codes_cols(hidden, elem)), dtype=np.uint8)
    scales = np.zeros((rows, hidden // BLOCK), dtype=np.uint8)
    rrms = np.zeros((rows,), dtype=np.float32)
    _check(lib().mxo_mxnorm_hadamard_fwd(_ptr(x, C.c_uint16), _ptr(g, C.c_uint16), rows,
                                         hidden, p, c, had, elem, _ptr(codes, C.c_uint8),
                                         _ptr(scales, C.c_uint8), _ptr(rrms, C.c_float)),
           "mxnorm_hadamard_fwd")
    return codes, scales, rrms


def rmsnorm_mxquant_fwd(x, gamma, eps, elem):
    x = _bf16(x)
    rows, hidden = x.shape
    g = None if gamma is None else _bf16(gamma)
    y = np.zeros((rows, hidden), dtype=np.uint16)
    codes = np.zeros((rows, codes_cols(hidden, elem)), dtype=np.uint8)
    scales = np.zeros((rows, hidden // BLOCK), dtype=np.uint8)
    rstd = np.zeros((rows,), dtype=np.float32)
    _check(lib().mxo_rmsnorm_mxquant_fwd(_ptr(x, C.c_uint16), _ptr(g, C.c_uint16), rows,
                                         hidden, eps, elem, _ptr(y, C.c_uint16),
                                         _ptr(codes, C.c_uint8), _ptr(scales, C.c_uint8),
                                         _ptr(rstd, C.c_float)), "rmsnorm_mxquant_fwd")
    return y, codes, scales, rstd


def max_threads():
    return lib().mxo_max_threads()


def set_threads(n):
    """Thread count of the oracle's OpenMP loops (for timing the CPU baseline)."""
    lib().mxo_set_threads(int(n))


def mxnorm_bwd(x, dy, gamma, rho):
    """Straight-through MXNorm backward (fp64, unrounded): returns (dx, dgamma);
    dgamma is None when gamma is None."""
    x = _bf16(x)
    dy = _bf16(dy)
    rows, hidden = x.shape
    assert dy.shape == x.shape
    g = None if gamma is None else _bf16(gamma)
    rho = np.ascontiguousarray(rho, dtype=np.float32)
    assert rho.shape == (rows,)
    dx = np.zeros((rows, hidden), dtype=np.float64)
    dgamma = None if g is None else np.zeros((hidden,), dtype=np.float64)
    _check(lib().mxo_mxnorm_bwd(_ptr(x, C.c_uint16), _ptr(dy, C.c_uint16), _ptr(g, C.c_uint16),
                                _ptr(rho, C.c_float), rows, hidden, _ptr(dx, C.c_double),
                                _ptr(dgamma, C.c_double)), "mxnorm_bwd")
    return dx, dgamma


def mxnorm_fwd_ex(x, gamma, p, c, source, had, elem):
    """Forward with either block-magnitude reading (and optional rotation)."""
    x = _bf16(x)
    rows, hidden = x.shape
    g = None if gamma is None else _bf16(gamma)
    codes = np.zeros((rows, codes_cols(hidden, elem)), dtype=np.uint8)
    scales = np.zeros((rows, hidden // BLOCK), dtype=np.uint8)
    rrms = np.zeros((rows,), dtype=np.float32)
    _check(lib().mxo_mxnorm_fwd_ex(_ptr(x, C.c_uint16), _ptr(g, C.c_uint16), rows, hidden, p, c,
                                   source, had, elem, _ptr(codes, C.c_uint8),
                                   _ptr(scales, C.c_uint8), _ptr(rrms, C.c_float)),
           "mxnorm_fwd_ex")
    return codes, scales, rrms


def row_stat_absmax(xrow, p):
    xrow = _bf16(xrow)
    E = C.c_int()
    S = C.c_uint64()
    _check(lib().mxo_row_stat_absmax(_ptr(xrow, C.c_uint16), xrow.size, p, C.byref(E),
                                     C.byref(S)), "row_stat_absmax")
    return E.value, S.value


def rho_absmax(E, S, K, p, c):
    return float(np.float32(lib().mxo_rho_absmax(E, S, K, p, c)))


def mx_quant_gain(w, gamma, elem):
    """MX cast of the gain-folded weight fl32(W * gamma) (MXNormLinear)."""
    w = _bf16(w)
    rows, hidden = w.shape
    g = _bf16(gamma)
    codes = np.zeros((rows, codes_cols(hidden, elem)), dtype=np.uint8)
    scales = np.zeros((rows, hidden // BLOCK), dtype=np.uint8)
    _check(lib().mxo_mx_quant_gain(_ptr(w, C.c_uint16), _ptr(g, C.c_uint16), rows, hidden, elem,
                                   _ptr(codes, C.c_uint8), _ptr(scales, C.c_uint8)),
           "mx_quant_gain")
    return codes, scales


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


def mx_matmul(a_codes, a_scales, b_codes, b_scales):
    """fp64 C = A B^T for MXFP8 (E4M3) A [M, K] and B [N, K]."""
    a_codes, a_scales, b_codes, b_scales = map(_u8, (a_codes, a_scales, b_codes, b_scales))
    M, K = a_codes.shape
    N = b_codes.shape[0]
    c = np.zeros((M, N), dtype=np.float64)
    _check(lib().mxo_mx_matmul(_ptr(a_codes, C.c_uint8), _ptr(a_scales, C.c_uint8),
                               _ptr(b_codes, C.c_uint8), _ptr(b_scales, C.c_uint8), M, N, K,
                               _ptr(c, C.c_double)), "mx_matmul")
    return c


def mx_matmul_sampled(a_codes, a_scales, b_codes, b_scales, mn):
    """fp64 C[m, n] for the listed (m, n) pairs only."""
    a_codes, a_scales, b_codes, b_scales = map(_u8, (a_codes, a_scales, b_codes, b_scales))
    K = a_codes.shape[1]
    mn = np.ascontiguousarray(mn, dtype=np.int64).reshape(-1, 2)
    out = np.zeros((mn.shape[0],), dtype=np.float64)
    _check(lib().mxo_mx_matmul_sampled(_ptr(a_codes, C.c_uint8), _ptr(a_scales, C.c_uint8),
                                       _ptr(b_codes, C.c_uint8), _ptr(b_scales, C.c_uint8), K,
                                       mn.ctypes.data_as(C.POINTER(C.c_int64)), mn.shape[0],
                                       _ptr(out, C.c_double)), "mx_matmul_sampled")
    return out
