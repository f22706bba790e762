"""MXNorm for AMD MI355X (gfx950): Python binding of libmxnorm.so.

Thin ctypes marshalling over the C ABI in ``include/mxnorm.h``: every step
of the computation runs in the library's HIP kernels.  PyTorch supplies
device memory and the current HIP stream; tensors in and out are
``torch.bfloat16`` (or int16/uint16 bit patterns) for bf16 data,
``torch.uint8`` for codes and scales, ``torch.float32`` for rrms / rstd.

The library is loaded from ``mx_quantised_tensor_amd/lib/libmxnorm.so``;
if it is missing, importing a kernel entry point raises -- there is no
fallback path.
"""
import ctypes as C
import os

import torch

__all__ = ["E4M3", "E2M1", "BLOCK", "MAX_HIDDEN", "MxqError", "lib", "mx_quant", "mxnorm_fwd",
           "mxnorm_bwd", "mxnorm_bwd_workspace_bytes", "mxnorm_bwd_noalloc", "mxnorm_fwd_ex", "SRC_SCALES",
           "SRC_ABSMAX", "OUT_F32", "OUT_BF16", "mx_quant_gain", "mx_matmul", "mxnorm_linear_fwd",
           "mxnorm_hadamard_fwd", "rmsnorm_mxquant_fwd", "mxnorm_default_c", "status_str",
           "library_path"]

E4M3 = 0
E2M1 = 1
BLOCK = 32
SRC_SCALES = 0   # block magnitude = the E8M0 scale as a power of two (mxnorm_fwd)
SRC_ABSMAX = 1   # block magnitude = the exact block absmax
OUT_F32 = 0      # matrix-product output types
OUT_BF16 = 1
MAX_HIDDEN = 32768

_HERE = os.path.dirname(os.path.abspath(__file__))
# MXQ_LIB overrides the path (e.g. a host-sanitizer build of the same sources)
_LIB_PATH = os.environ.get("MXQ_LIB") or os.path.join(_HERE, "lib", "libmxnorm.so")
_lib = None

EXPORTED = ("mx_quant", "mxnorm_fwd", "mxnorm_hadamard_fwd", "rmsnorm_mxquant_fwd",
            "mxnorm_default_c", "mxq_status_str", "mxq_version")


class MxqError(RuntimeError):
    pass


def library_path():
    return _LIB_PATH


def lib():
    """Load libmxnorm.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MxqError("libmxnorm.so not built: run __graft_entry__.build() or "
                           "python mx_quantised_tensor_amd/build.py (looked for %s)" % _LIB_PATH)
        L = C.CDLL(_LIB_PATH)
        vp, i64, i32, f32 = C.c_void_p, C.c_int64, C.c_int, C.c_float
        L.mx_quant.restype = i32
        L.mx_quant.argtypes = [vp, i64, i64, i32, vp, vp, vp]
        L.mxnorm_fwd.restype = i32
        L.mxnorm_fwd.argtypes = [vp, vp, i64, i64, i32, f32, i32, vp, vp, vp, vp]
        L.mxnorm_hadamard_fwd.restype = i32
        L.mxnorm_hadamard_fwd.argtypes = [vp, vp, i64, i64, i32, f32, i32, i32, vp, vp, vp, vp]
        L.rmsnorm_mxquant_fwd.restype = i32
        L.rmsnorm_mxquant_fwd.argtypes = [vp, vp, i64, i64, f32, i32, vp, vp, vp, vp, vp]
        L.mxnorm_bwd.restype = i32
        L.mxnorm_bwd.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp, vp, vp]
        L.mxnorm_bwd_workspace_bytes.restype = C.c_size_t
        L.mxnorm_bwd_workspace_bytes.argtypes = [i64, i64]
        L.mxnorm_bwd_noalloc.restype = i32
        L.mxnorm_bwd_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp, vp]
        L.mxnorm_bwd_noalloc_scratch_bytes.restype = C.c_size_t
        L.mxnorm_bwd_noalloc_scratch_bytes.argtypes = []
        L.mx_quant_gain.restype = i32
        L.mx_quant_gain.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp]
        L.mx_matmul.restype = i32
        L.mx_matmul.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, vp]
        L.mxnorm_linear_fwd.restype = i32
        L.mxnorm_linear_fwd.argtypes = [vp, i64, i64, i32, f32, vp, vp, i64, vp, vp, vp, vp, i32,
                                        vp]
        L.mxnorm_fwd_ex.restype = i32
        L.mxnorm_fwd_ex.argtypes = [vp, vp, i64, i64, i32, f32, i32, i32, i32, vp, vp, vp, vp]
        L.mxnorm_default_c_for.restype = f32
        L.mxnorm_default_c_for.argtypes = [i32, i32]
        L.mxnorm_default_c.restype = f32
        L.mxnorm_default_c.argtypes = [i32]
        L.mxq_status_str.restype = C.c_char_p
        L.mxq_status_str.argtypes = [i32]
        L.mxq_version.restype = C.c_char_p
        L.mxq_version.argtypes = []
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().mxq_status_str(status).decode()


def mxnorm_default_c(p: int, source: int = SRC_SCALES) -> float:
    return float(lib().mxnorm_default_c_for(int(p), int(source)))


def _check(status: int, name: str):
    if status != 0:
        raise MxqError("%s failed: %s" % (name, status_str(status)))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _bf16_2d(x):
    if x.dim() != 2:
        raise ValueError("expected a 2-D [rows, hidden] tensor")
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("bf16 data must be torch.bfloat16 (or 16-bit integer bit patterns)")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    return x


def _gamma(g, hidden):
    if g is None:
        return None
    if g.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or g.numel() != hidden:
        raise ValueError("gamma must be bf16 with `hidden` elements")
    if not g.is_cuda or not g.is_contiguous():
        raise ValueError("gamma must be a contiguous device tensor")
    return g


def _outputs(x, elem, codes, scales):
    rows, hidden = x.shape
    ccols = hidden if elem == E4M3 else hidden // 2
    if codes is None:
        codes = torch.empty((rows, ccols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, hidden // BLOCK), dtype=torch.uint8, device=x.device)
    if codes.numel() != rows * ccols or scales.numel() != rows * (hidden // BLOCK):
        raise ValueError("codes / scales have the wrong size")
    return codes, scales


def mx_quant(x, elem=E4M3, codes=None, scales=None, stream=None):
    """MX cast of bf16 x [rows, hidden] -> (codes, scales)."""
    x = _bf16_2d(x)
    rows, hidden = x.shape
    codes, scales = _outputs(x, elem, codes, scales)
    _check(lib().mx_quant(_ptr(x), rows, hidden, elem, _ptr(codes), _ptr(scales),
                          _stream(stream)), "mx_quant")
    return codes, scales


def mxnorm_fwd(x, gamma=None, p=2, c=0.0, elem=E4M3, codes=None, scales=None, rrms=None,
               want_rrms=True, stream=None):
    """MXNorm forward -> (codes, scales, rrms).  c = 0 selects the default c(p)."""
    x = _bf16_2d(x)
    rows, hidden = x.shape
    gamma = _gamma(gamma, hidden)
    codes, scales = _outputs(x, elem, codes, scales)
    if rrms is None and want_rrms:
        rrms = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().mxnorm_fwd(_ptr(x), _ptr(gamma), rows, hidden, p, c, elem, _ptr(codes),
                            _ptr(scales), _ptr(rrms), _stream(stream)), "mxnorm_fwd")
    return codes, scales, rrms


def mxnorm_hadamard_fwd(x, gamma=None, p=2, c=0.0, had=16, elem=E2M1, codes=None, scales=None,
                        rrms=None, want_rrms=True, stream=None):
    """MXNorm forward with an H16/H32 rotation before the cast."""
    x = _bf16_2d(x)
    rows, hidden = x.shape
    gamma = _gamma(gamma, hidden)
    codes, scales = _outputs(x, elem, codes, scales)
    if rrms is None and want_rrms:
        rrms = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().mxnorm_hadamard_fwd(_ptr(x), _ptr(gamma), rows, hidden, p, c, had, elem,
                                     _ptr(codes), _ptr(scales), _ptr(rrms), _stream(stream)),
           "mxnorm_hadamard_fwd")
    return codes, scales, rrms


def mxnorm_fwd_ex(x, gamma=None, p=2, c=0.0, source=SRC_SCALES, had=0, elem=E4M3, codes=None,
                  scales=None, rrms=None, want_rrms=True, stream=None):
    """MXNorm forward with a choice of block magnitude (and optional rotation)."""
    x = _bf16_2d(x)
    rows, hidden = x.shape
    gamma = _gamma(gamma, hidden)
    codes, scales = _outputs(x, elem, codes, scales)
    if rrms is None and want_rrms:
        rrms = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().mxnorm_fwd_ex(_ptr(x), _ptr(gamma), rows, hidden, p, c, source, had, elem,
                               _ptr(codes), _ptr(scales), _ptr(rrms), _stream(stream)),
           "mxnorm_fwd_ex")
    return codes, scales, rrms


def rmsnorm_mxquant_fwd(x, gamma=None, eps=1e-5, elem=E4M3, y=None, codes=None, scales=None,
                        rstd=None, want_rstd=True, stream=None):
    """Two-pass baseline: RMSNorm to bf16 y, then mx_quant(y) -> (y, codes, scales, rstd)."""
    x = _bf16_2d(x)
    rows, hidden = x.shape
    gamma = _gamma(gamma, hidden)
    codes, scales = _outputs(x, elem, codes, scales)
    if y is None:
        y = torch.empty((rows, hidden), dtype=torch.bfloat16, device=x.device)
    if rstd is None and want_rstd:
        rstd = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().rmsnorm_mxquant_fwd(_ptr(x), _ptr(gamma), rows, hidden, eps, elem, _ptr(y),
                                     _ptr(codes), _ptr(scales), _ptr(rstd), _stream(stream)),
           "rmsnorm_mxquant_fwd")
    return y, codes, scales, rstd


def mxnorm_bwd_workspace_bytes(rows: int, hidden: int) -> int:
    return int(lib().mxnorm_bwd_workspace_bytes(rows, hidden))


def mxnorm_bwd(x, dy, rrms, gamma=None, dx=None, dgamma=None, workspace=None, stream=None):
    """Straight-through MXNorm backward -> (dx bf16, dgamma fp32 or None).

    x, dy: bf16 [rows, hidden]; rrms: fp32 [rows] from the forward.  The
    workspace (needed with a gain) is allocated here unless one is passed."""
    x = _bf16_2d(x)
    dy = _bf16_2d(dy)
    rows, hidden = x.shape
    if tuple(dy.shape) != (rows, hidden):
        raise ValueError("dy must have the shape of x")
    if rrms.dtype != torch.float32 or rrms.numel() != rows or not rrms.is_cuda:
        raise ValueError("rrms must be a device fp32 tensor with one value per row")
    gamma = _gamma(gamma, hidden)
    if dx is None:
        dx = torch.empty((rows, hidden), dtype=torch.bfloat16, device=x.device)
    if gamma is not None:
        if dgamma is None:
            dgamma = torch.empty((hidden,), dtype=torch.float32, device=x.device)
        if workspace is None:
            nbytes = mxnorm_bwd_workspace_bytes(rows, hidden)
            workspace = torch.empty((max(nbytes, 16) // 4,), dtype=torch.float32,
                                    device=x.device)
    else:
        dgamma = None
    _check(lib().mxnorm_bwd(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(rrms), rows, hidden, _ptr(dx),
                            _ptr(dgamma), _ptr(workspace), _stream(stream)), "mxnorm_bwd")
    return dx, dgamma


def mxnorm_bwd_noalloc(x, dy, rrms, gamma=None, dx=None, dgamma=None, stream=None):
    """mxnorm_bwd with the library's static per-GPU scratch instead of a
    workspace (the C call allocates nothing; pass dx / dgamma to allocate
    nothing here either).  Calls overlapping on one GPU race."""
    x = _bf16_2d(x)
    dy = _bf16_2d(dy)
    rows, hidden = x.shape
    if tuple(dy.shape) != (rows, hidden):
        raise ValueError("dy must have the shape of x")
    if rrms.dtype != torch.float32 or rrms.numel() != rows or not rrms.is_cuda:
        raise ValueError("rrms must be a device fp32 tensor with one value per row")
    gamma = _gamma(gamma, hidden)
    if dx is None:
        dx = torch.empty((rows, hidden), dtype=torch.bfloat16, device=x.device)
    if gamma is not None:
        if dgamma is None:
            dgamma = torch.empty((hidden,), dtype=torch.float32, device=x.device)
    else:
        dgamma = None
    _check(lib().mxnorm_bwd_noalloc(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(rrms), rows, hidden,
                                    _ptr(dx), _ptr(dgamma), _stream(stream)),
           "mxnorm_bwd_noalloc")
    return dx, dgamma


def mx_quant_gain(w, gamma, elem=E4M3, codes=None, scales=None, stream=None):
    """MX cast of the gain-folded weight fl32(W * gamma) -> (codes, scales)."""
    w = _bf16_2d(w)
    rows, hidden = w.shape
    gamma = _gamma(gamma, hidden)
    if gamma is None:
        raise ValueError("mx_quant_gain needs a gain")
    codes, scales = _outputs(w, elem, codes, scales)
    _check(lib().mx_quant_gain(_ptr(w), _ptr(gamma), rows, hidden, elem, _ptr(codes),
                               _ptr(scales), _stream(stream)), "mx_quant_gain")
    return codes, scales


def _u8_2d(t, name):
    if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous 2-D uint8 device tensor" % name)
    return t


def _out_type(t, name):
    """mxq_out code of an output tensor's dtype (fp32 or bf16)."""
    if t.dtype == torch.float32:
        return OUT_F32
    if t.dtype == torch.bfloat16:
        return OUT_BF16
    raise ValueError("%s must be float32 or bfloat16" % name)


def mx_matmul(a_codes, a_scales, b_codes, b_scales, c=None, out_dtype=torch.float32, stream=None):
    """C = A B^T for MXFP8 A [M, K] and B [N, K]; C fp32, or bf16 (the fp32
    result rounded to nearest even) -- the dtype of c if given, else out_dtype."""
    a_codes, a_scales = _u8_2d(a_codes, "a_codes"), _u8_2d(a_scales, "a_scales")
    b_codes, b_scales = _u8_2d(b_codes, "b_codes"), _u8_2d(b_scales, "b_scales")
    M, K = a_codes.shape
    N = b_codes.shape[0]
    if b_codes.shape[1] != K or a_scales.shape != (M, K // BLOCK) or \
            b_scales.shape != (N, K // BLOCK):
        raise ValueError("operand shapes do not agree")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    _check(lib().mx_matmul(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K,
                           _ptr(c), _out_type(c, "c"), _stream(stream)), "mx_matmul")
    return c


def mxnorm_linear_fwd(x, w_codes, w_scales, p=2, c=0.0, out=None, x_codes=None, x_scales=None,
                      rrms=None, out_dtype=torch.float32, stream=None):
    """MXNormLinear forward: mxnorm_fwd (no gain, E4M3) then mx_matmul with the
    gain-folded MXFP8 weight -> (out [rows, out_features] fp32 or bf16, x_codes,
    x_scales, rrms)."""
    x = _bf16_2d(x)
    rows, hidden = x.shape
    w_codes, w_scales = _u8_2d(w_codes, "w_codes"), _u8_2d(w_scales, "w_scales")
    O = w_codes.shape[0]
    x_codes, x_scales = _outputs(x, E4M3, x_codes, x_scales)
    if rrms is None:
        rrms = torch.empty((rows,), dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty((rows, O), dtype=out_dtype, device=x.device)
    _check(lib().mxnorm_linear_fwd(_ptr(x), rows, hidden, p, c, _ptr(w_codes), _ptr(w_scales), O,
                                   _ptr(x_codes), _ptr(x_scales), _ptr(rrms), _ptr(out),
                                   _out_type(out, "out"), _stream(stream)), "mxnorm_linear_fwd")
    return out, x_codes, x_scales, rrms
