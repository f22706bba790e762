"""GPU tests: library calls captured in a HIP graph, the way a caller under
graph capture uses them, then replayed several times.  Between replays
eager work overwrites every output buffer.  Each replay must reproduce
the eager call's bits exactly.

A call only launches kernels: it allocates nothing, clears nothing with a
memset, and never synchronises, so a captured call is the same work as
an eager one.  The outputs' bits are compared byte by byte."""
import pytest
import torch

import mx_quantised_tensor_amd as mxq
from mx_quantised_tensor_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    mxq.lib()
    yield


def _bytes(t):
    return t.contiguous().view(torch.uint8).reshape(-1).clone()


def _check_replays(run, outs, what):
    print("case:", what, flush=True)
    run()
    torch.cuda.synchronize()
    ref = [_bytes(o) for o in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        run()
    torch.cuda.synchronize()
    for k in range(REPLAYS):
        for o in outs:  # eager work on the same buffers between replays
            o.view(torch.uint8).fill_(0xA5 if k % 2 == 0 else 0x3C)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bytes(o), r), "%s: replay %d, output %d differs" % (what, k, i)
    del graph


def _inputs(rows, hidden, seed, kind="rowscale"):
    xb, gb = W.generate(rows, hidden, kind, seed)
    return P.to_device_bf16(xb), P.to_device_bf16(gb)


@pytest.mark.parametrize("rows,hidden,elem", [(8192, 2048, 0), (8192, 4096, 0), (8192, 4096, 1),
                                              (300, 768, 0)])
def test_graph_mxnorm_fwd(rows, hidden, elem):
    # the 2048-column kernel with its 4-wave part, the 2-wave rows with
    # theirs, E2M1, and a short launch
    x, g = _inputs(rows, hidden, rows + hidden)
    codes, scales, rho = mxq.mxnorm_fwd(x, g, p=2, elem=elem)
    _check_replays(lambda: mxq.mxnorm_fwd(x, g, p=2, elem=elem, codes=codes, scales=scales,
                                          rrms=rho),
                   [codes, scales, rho], "mxnorm_fwd %dx%d elem=%d" % (rows, hidden, elem))


@pytest.mark.parametrize("had,elem", [(16, 1), (32, 0)])
def test_graph_hadamard(had, elem):
    x, g = _inputs(1024, 4096, had + elem)
    codes, scales, rho = mxq.mxnorm_hadamard_fwd(x, g, had=had, elem=elem)
    _check_replays(lambda: mxq.mxnorm_hadamard_fwd(x, g, had=had, elem=elem, codes=codes,
                                                   scales=scales, rrms=rho),
                   [codes, scales, rho], "mxnorm_hadamard_fwd H%d elem=%d" % (had, elem))


def test_graph_two_pass_baseline():
    x, g = _inputs(1024, 4096, 5)
    y = torch.empty_like(x)
    _, codes, scales, rstd = mxq.rmsnorm_mxquant_fwd(x, g, y=y)
    _check_replays(lambda: mxq.rmsnorm_mxquant_fwd(x, g, y=y, codes=codes, scales=scales,
                                                   rstd=rstd),
                   [y, codes, scales, rstd], "rmsnorm_mxquant_fwd 1024x4096")


@pytest.mark.parametrize("rows,hidden,with_gamma", [(4096, 4096, True), (16384, 4096, False),
                                                    (1000, 8192, True), (300, 32768, True),
                                                    (2000, 1024, True)])
def test_graph_mxnorm_bwd(rows, hidden, with_gamma):
    # the persistent row kernels and the dgamma column sum (two launches),
    # and the no-gain layouts
    x, g = _inputs(rows, hidden, rows + 3)
    dy = P.to_device_bf16(W.grad_output(rows, hidden, rows + 4))
    _, _, rho = mxq.mxnorm_fwd(x, g, p=2)
    gg = g if with_gamma else None
    dx, dg = mxq.mxnorm_bwd(x, dy, rho, gg)
    ws = None
    if with_gamma:
        nb = mxq.mxnorm_bwd_workspace_bytes(rows, hidden)
        ws = torch.empty((max(nb, 16) // 4,), dtype=torch.float32, device="cuda")
    outs = [dx] + ([dg] if with_gamma else [])
    _check_replays(lambda: mxq.mxnorm_bwd(x, dy, rho, gg, dx=dx, dgamma=dg, workspace=ws),
                   outs, "mxnorm_bwd %dx%d gamma=%s" % (rows, hidden, with_gamma))


def test_graph_mxnorm_bwd_noalloc():
    rows, hidden = 2048, 8192
    x, g = _inputs(rows, hidden, 77)
    dy = P.to_device_bf16(W.grad_output(rows, hidden, 78))
    _, _, rho = mxq.mxnorm_fwd(x, g, p=2)
    dx, dg = mxq.mxnorm_bwd_noalloc(x, dy, rho, g)
    _check_replays(lambda: mxq.mxnorm_bwd_noalloc(x, dy, rho, g, dx=dx, dgamma=dg), [dx, dg],
                   "mxnorm_bwd_noalloc %dx%d" % (rows, hidden))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_graph_matmul(out_dtype):
    x, g = _inputs(512, 1024, 9)
    w = (torch.randn(1024, 1024, generator=torch.Generator().manual_seed(9)) / 32).to(
        torch.bfloat16).cuda()
    wc, ws = mxq.mx_quant_gain(w, g)
    xc, xs, _ = mxq.mxnorm_fwd(x, None, p=2)
    out = mxq.mx_matmul(xc, xs, wc, ws, out_dtype=out_dtype)
    _check_replays(lambda: mxq.mx_matmul(xc, xs, wc, ws, c=out), [out],
                   "mx_matmul 512x1024x1024 %s" % out_dtype)


def test_graph_forward_then_backward_chain():
    # one graph holding the forward and the backward that uses its rho
    rows, hidden = 4096, 4096
    x, g = _inputs(rows, hidden, 123)
    dy = P.to_device_bf16(W.grad_output(rows, hidden, 124))
    codes, scales, rho = mxq.mxnorm_fwd(x, g, p=2)
    dx, dg = mxq.mxnorm_bwd(x, dy, rho, g)
    nb = mxq.mxnorm_bwd_workspace_bytes(rows, hidden)
    ws = torch.empty((max(nb, 16) // 4,), dtype=torch.float32, device="cuda")

    def run():
        mxq.mxnorm_fwd(x, g, p=2, codes=codes, scales=scales, rrms=rho)
        mxq.mxnorm_bwd(x, dy, rho, g, dx=dx, dgamma=dg, workspace=ws)

    _check_replays(run, [codes, scales, rho, dx, dg], "forward then backward 4096x4096")
