"""GPU test of mxnorm_bwd_noalloc (the backward for callers that cannot
allocate: its workspace is the library's static per-GPU scratch array),
through the C ABI, against mxnorm_bwd with a caller-owned workspace: dx and
dgamma must be bit-identical (same kernels, same summation order), and both
within the fp64 oracle's bar.  Two calls in a row, the second with a smaller
input, so the second runs on a scratch array that still holds the first
call's partial rows."""
import ctypes as C

import numpy as np
import pytest
import torch

import mx_quantised_tensor_amd as mxq
import oracle as O
from mx_quantised_tensor_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

C2 = float.fromhex("0x1.c1ed54p+0")


def _case(rows, hidden, seed):
    xb, gb = W.generate(rows, hidden, "rowscale", seed)
    dyb = W.grad_output(rows, hidden, seed)
    _, _, rho = O.mxnorm_fwd(xb, gb, 2, C2, O.E4M3)
    return xb, dyb, gb, rho


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _call_both(xb, dyb, gb, rho, with_gamma):
    L = mxq.lib()
    rows, hidden = xb.shape
    x, dy = P.to_device_bf16(xb), P.to_device_bf16(dyb)
    g = P.to_device_bf16(gb) if with_gamma else None
    r = torch.from_numpy(np.ascontiguousarray(rho)).cuda()
    sp = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for noalloc in (True, False):
        dx = torch.full((rows, hidden), 7.0, dtype=torch.bfloat16, device="cuda")
        dg = torch.full((hidden,), 7.0, dtype=torch.float32, device="cuda") if with_gamma else None
        if noalloc:
            rc = L.mxnorm_bwd_noalloc(_ptr(x), _ptr(dy), _ptr(g), _ptr(r), rows, hidden, _ptr(dx),
                                      _ptr(dg), sp)
        else:
            nb = mxq.mxnorm_bwd_workspace_bytes(rows, hidden)
            ws = torch.empty((max(nb, 16) // 4,), dtype=torch.float32, device="cuda")
            rc = L.mxnorm_bwd(_ptr(x), _ptr(dy), _ptr(g), _ptr(r), rows, hidden, _ptr(dx),
                              _ptr(dg), _ptr(ws) if with_gamma else None, sp)
        assert rc == 0, mxq.status_str(rc)
        torch.cuda.synchronize()
        out.append((P.from_device(dx.view(torch.int16)).view(np.uint16),
                    None if dg is None else P.from_device(dg)))
    return out


@pytest.mark.parametrize("first,second", [((3000, 8192), (37, 1024)),
                                          ((300, 32768), (5, 4096)),
                                          ((1000, 4096), (3, 96))])
@pytest.mark.parametrize("with_gamma", [True, False])
def test_noalloc_matches_workspace_entry_point(first, second, with_gamma):
    assert mxq.lib().mxnorm_bwd_noalloc_scratch_bytes() == 32 << 20
    for k, (rows, hidden) in enumerate((first, second)):
        what = "noalloc call %d rows=%d hidden=%d gamma=%s" % (k + 1, rows, hidden, with_gamma)
        print("case:", what, flush=True)
        xb, dyb, gb, rho = _case(rows, hidden, 100 + k)
        (dx_n, dg_n), (dx_w, dg_w) = _call_both(xb, dyb, gb, rho, with_gamma)
        assert np.array_equal(dx_n, dx_w), what + ": dx differs from mxnorm_bwd"
        if with_gamma:
            assert np.array_equal(dg_n.view(np.uint32), dg_w.view(np.uint32)), \
                what + ": dgamma differs from mxnorm_bwd"
        ref_dx, ref_dg = O.mxnorm_bwd(xb, dyb, gb if with_gamma else None, rho)
        P.assert_bwd_close(dx_n, dg_n, xb, dyb, gb if with_gamma else None, rho, ref_dx,
                           ref_dg if with_gamma else None, what)
