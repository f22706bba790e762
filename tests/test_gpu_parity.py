"""GPU parity: libmxnorm.so (through its C ABI) against the CPU oracle, on
the same seeded inputs.  Run on an MI355X with ``pytest -m gpu``.

Bars (see tests/parity.py): E8M0 scales byte-equal and rho bit-equal always;
MXNorm / mx_quant / Hadamard element codes are required to be identical (the
acceptance bar allows one step on 0.01% of elements; these kernels are held
to zero).  The two-pass baseline accumulates its sum of squares in fp32 on
the GPU and in fp64 in the oracle, so it is held to: rstd rel <= 1e-5, bf16 y
within one bf16 ulp, codes within one step on <= 0.01% of elements, scales
differing on <= 0.01% of blocks and then by one.
"""
import numpy as np
import pytest
import torch

import mx_quantised_tensor_amd as mxq
import oracle as O
from mx_quantised_tensor_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

C_DEF = {1: float.fromhex("0x1.b16c5ep+0"), 2: float.fromhex("0x1.c1ed54p+0")}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    mxq.lib()
    yield


def _run_mxnorm(xb, gb, p, c, elem, had=0):
    x = P.to_device_bf16(xb)
    g = None if gb is None else P.to_device_bf16(gb)
    if had:
        codes, scales, rho = mxq.mxnorm_hadamard_fwd(x, g, p=p, c=c, had=had, elem=elem)
    else:
        codes, scales, rho = mxq.mxnorm_fwd(x, g, p=p, c=c, elem=elem)
    torch.cuda.synchronize()
    return P.from_device(codes), P.from_device(scales), P.from_device(rho)


def _check_mxnorm(xb, gb, p, c, elem, had=0, what=""):
    gc, gs, gr = _run_mxnorm(xb, gb, p, c, elem, had)
    if had:
        oc, os_, orr = O.mxnorm_hadamard_fwd(xb, gb, p, c, had, elem)
    else:
        oc, os_, orr = O.mxnorm_fwd(xb, gb, p, c, elem)
    P.assert_rho_equal(gr, orr, what)
    P.assert_scales_equal(gs, os_, what)
    P.assert_codes(gc, oc, os_, elem, exact=True, what=what)


def _bits(a):
    return W.to_bf16_bits(np.asarray(a, dtype=np.float32))


# ------------------------------------------------------------------- mx_quant

@pytest.mark.parametrize("elem", [0, 1])
@pytest.mark.parametrize("hidden", [32, 96, 768, 4096, 4128, 32768])
@pytest.mark.parametrize("rows", [1, 3, 130])
def test_mx_quant_shapes(elem, hidden, rows):
    xb, _ = W.generate(rows, hidden, "t3", seed=hidden + rows)
    codes, scales = mxq.mx_quant(P.to_device_bf16(xb), elem=elem)
    torch.cuda.synchronize()
    oc, os_ = O.mx_quant(xb, elem)
    P.assert_scales_equal(P.from_device(scales), os_, "mx_quant")
    P.assert_codes(P.from_device(codes), oc, os_, elem, exact=True, what="mx_quant")


def _edge_matrix():
    rng = np.random.default_rng(99)
    rows = []
    rows.append(np.zeros(64))                                   # zeros
    rows.append(-np.zeros(64))                                  # negative zeros
    rows.append(rng.standard_normal(64) * 1e-39)                # bf16 subnormals
    rows.append(rng.standard_normal(64) * 1e38)                 # near the top of bf16
    r = rng.standard_normal(64); r[5] = np.inf; rows.append(r)  # Inf in block 0
    r = rng.standard_normal(64); r[40] = np.nan; rows.append(r) # NaN in block 1
    # saturation: block max 1.9375 * 2^k -> 496 after the scale, clamps to 448
    r = rng.uniform(-1, 1, 64); r[0] = 1.9375; r[33] = -1.96875 * 1024; rows.append(r)
    # ties: values on E4M3 midpoints after scaling by 2^(0-8)
    r = np.array([1.0] + [(2 ** -8) * (m + 0.5) / 8 * 2 ** 1 for m in range(31)] +
                 [1.0] + [(2 ** -5) * (1 + (m % 8 + 0.5) / 8) for m in range(31)])
    rows.append(r)
    rows.append(np.full(64, 3.0))
    rows.append(np.where(np.arange(64) % 2 == 0, 6.5, -0.25))  # E2M1 saturation and ties
    return _bits(np.array(rows))


@pytest.mark.parametrize("elem", [0, 1])
def test_mx_quant_edge_values(elem):
    xb = _edge_matrix()
    codes, scales = mxq.mx_quant(P.to_device_bf16(xb), elem=elem)
    torch.cuda.synchronize()
    oc, os_ = O.mx_quant(xb, elem)
    P.assert_scales_equal(P.from_device(scales), os_, "mx_quant edge")
    P.assert_codes(P.from_device(codes), oc, os_, elem, exact=True, what="mx_quant edge")


# ------------------------------------------------------------------ MXNorm

@pytest.mark.parametrize("cfg,p", [(1, 2), (2, 1), (2, 2), (3, 2), (4, 2)])
def test_mxnorm_workloads_full(cfg, p):
    w = W.WORKLOADS[cfg]
    xb, gb = W.workload_inputs(cfg)
    print("workload", w.name, "p", p, flush=True)
    _check_mxnorm(xb, gb, p, C_DEF[p], w.elem, w.had, what=w.name)


@pytest.mark.parametrize("hidden", [32, 64, 96, 160, 512, 768, 1056, 2048, 2080, 2560, 2592, 3072,
                                    3104, 4064, 4096, 4128, 5120, 5152, 6144, 6176, 7168, 7200,
                                    8192, 10240, 10272, 12288, 14336, 16384, 20480, 20512,
                                    24576, 28672, 28704, 32768])
@pytest.mark.parametrize("elem", [0, 1])
def test_mxnorm_shapes(hidden, elem):
    rows = 67 if hidden <= 8192 else 9
    xb, gb = W.generate(rows, hidden, "rowscale", seed=hidden * 3 + elem)
    for p in (1, 2):
        _check_mxnorm(xb, gb, p, C_DEF[p], elem, what="D=%d p=%d" % (hidden, p))
        _check_mxnorm(xb, None, p, 1.25, elem, what="D=%d p=%d no gamma" % (hidden, p))


@pytest.mark.parametrize("rows", [1, 2, 3, 5, 255, 257])
def test_mxnorm_ragged_row_counts(rows):
    xb, gb = W.generate(rows, 2048, "outlier", seed=rows)
    _check_mxnorm(xb, gb, 2, C_DEF[2], 0, what="rows=%d" % rows)


@pytest.mark.parametrize("hidden,had", [(4096, 0), (4096, 16), (4096, 32), (2048, 0), (8192, 0)])
@pytest.mark.parametrize("elem", [0, 1])
def test_mxnorm_scales_at_odd_address(hidden, had, elem):
    """Scale bytes written one byte at a time when the scales buffer is not
    4-byte aligned (every kernel has that path beside its dword stores)."""
    rows = 13
    xb, gb = W.generate(rows, hidden, "outlier", seed=hidden + had + elem)
    x = P.to_device_bf16(xb)
    g = P.to_device_bf16(gb)
    k = hidden // 32
    buf = torch.full((rows * k + 1,), 0x5A, dtype=torch.uint8, device="cuda")
    scales = buf[1:]
    print("case: hidden=%d had=%d elem=%d scales at +1" % (hidden, had, elem), flush=True)
    if had:
        codes, _, rho = mxq.mxnorm_hadamard_fwd(x, g, p=2, c=C_DEF[2], had=had, elem=elem,
                                                scales=scales)
        oc, os_, orr = O.mxnorm_hadamard_fwd(xb, gb, 2, C_DEF[2], had, elem)
    else:
        codes, _, rho = mxq.mxnorm_fwd(x, g, p=2, c=C_DEF[2], elem=elem, scales=scales)
        oc, os_, orr = O.mxnorm_fwd(xb, gb, 2, C_DEF[2], elem)
    torch.cuda.synchronize()
    what = "D=%d H%d elem=%d odd scales" % (hidden, had, elem)
    assert int(buf[0].item()) == 0x5A, "byte before the scales was written"
    gs = P.from_device(scales).reshape(rows, k)
    P.assert_rho_equal(P.from_device(rho), orr, what)
    P.assert_scales_equal(gs, os_, what)
    P.assert_codes(P.from_device(codes), oc, os_, elem, exact=True, what=what)


def _edge_rows(hidden):
    rng = np.random.default_rng(7)
    base = rng.standard_normal(hidden)
    rows = [np.zeros(hidden), -np.zeros(hidden), base * 1e-39, base * 3e37, base * 1e-30]
    r = base.copy(); r[3] = np.nan; rows.append(r)
    r = base.copy(); r[hidden - 1] = -np.inf; rows.append(r)
    r = np.zeros(hidden); r[0] = 1.0; rows.append(r)
    r = np.zeros(hidden); r[hidden // 2] = 2.0 ** -124; rows.append(r)   # large rho
    r = np.full(hidden, 1.5 * 2.0 ** 126); rows.append(r)               # rho near 2^-127
    r = base * 2.0 ** 100; r[::32] = 3e38; rows.append(r)
    return _bits(np.array(rows))


@pytest.mark.parametrize("elem", [0, 1])
@pytest.mark.parametrize("p", [1, 2])
@pytest.mark.parametrize("hidden", [64, 4096])
def test_mxnorm_edge_rows(elem, p, hidden):
    xb = _edge_rows(hidden)
    gb = _bits(1 + 0.02 * np.random.default_rng(3).standard_normal(hidden))
    for c in (0.3, 1.0, C_DEF[p], 3.5, 10.0):  # 0.3: subnormal rho; 10: rho overflow
        _check_mxnorm(xb, gb, p, c, elem, what="edge c=%g" % c)
        _check_mxnorm(xb, None, p, c, elem, what="edge no gamma c=%g" % c)


@pytest.mark.parametrize("rows,hidden", [(r, h) for r in (8191, 8192, 8193, 10001)
                                         for h in (3072, 4064, 4096)] +
                         [(r, h) for r in (8192, 8193) for h in (4608, 5152, 6144, 8192)])
def test_mxnorm_wide_tail_part(rows, hidden):
    """E4M3 launches of 8192 rows or more with rows of 2 waves of 4 to 8
    steps (3072 < hidden <= 8192) hand their last 2048 rows to workgroups of
    one row and 4 waves of half as many steps (3072: 3 steps, no tail part):
    the boundary between the two parts (odd row counts leave the last 2-row
    workgroup half empty), ragged widths (4064; 4608 and 5152: 5 and 6 steps
    with a ragged last one, the tail part's last step past the row end), and
    edge rows placed in the tail part."""
    xb, gb = W.generate(rows, hidden, "rowscale", seed=rows + hidden)
    e = _edge_rows(hidden)
    xb[rows - 1 - len(e):rows - 1] = e          # in the tail part
    xb[rows - 2048 - 3:rows - 2048 + 3] = e[:6]  # across the boundary
    for p, c in ((2, C_DEF[2]), (1, 0.3)):
        _check_mxnorm(xb, gb, p, c, 0, what="tail rows=%d D=%d p=%d" % (rows, hidden, p))
    _check_mxnorm(xb, None, 2, 10.0, 0, what="tail rows=%d D=%d no gamma" % (rows, hidden))


@pytest.mark.parametrize("rows", [8191, 8192, 8193, 9999])
def test_mxnorm_wave_tail_part(rows):
    """E4M3 launches of 8192 rows or more at hidden 2048 (one wave per row)
    hand their last 1536 rows to workgroups of one row and 4 waves: the
    boundary between the two parts (row counts that leave the last 4-row
    workgroup partly empty), 8191 rows (no tail part), and edge rows placed
    in the tail part."""
    hidden = 2048
    xb, gb = W.generate(rows, hidden, "rowscale", seed=rows + 11)
    e = _edge_rows(hidden)
    xb[rows - 1 - len(e):rows - 1] = e          # in the tail part
    xb[rows - 1536 - 3:rows - 1536 + 3] = e[:6]  # across the boundary
    for p, c in ((2, C_DEF[2]), (1, 0.3)):
        _check_mxnorm(xb, gb, p, c, 0, what="wave tail rows=%d p=%d" % (rows, p))
    _check_mxnorm(xb, None, 2, 10.0, 0, what="wave tail rows=%d no gamma" % rows)
    _check_mxnorm(xb, gb, 2, C_DEF[2], 1, what="wave tail rows=%d E2M1 (no tail)" % rows)


def test_mxnorm_wide_tail_part_sampled():
    # a large E4M3 launch at hidden 4096 (the head part 292 K workgroups, then
    # 2048 one-row workgroups), checked on sampled rows the oracle computes one
    # by one, every row around the boundary of the two parts included
    rows, hidden = 600001, 4096
    gen = torch.Generator(device="cuda")
    gen.manual_seed(37)
    x = (torch.randn(rows, hidden, device="cuda", generator=gen) * 2.0).to(torch.bfloat16)
    g = (1 + 0.02 * torch.randn(hidden, device="cuda", generator=gen)).to(torch.bfloat16)
    print("case: mxnorm_fwd rows=%d hidden=%d" % (rows, hidden), flush=True)
    codes, scales, rho = mxq.mxnorm_fwd(x, g, p=2, c=C_DEF[2], elem=O.E4M3)
    torch.cuda.synchronize()
    rng = np.random.default_rng(37)
    b = rows - 2048
    idx = np.unique(np.concatenate([rng.integers(0, rows, 1500), np.arange(b - 4, b + 4),
                                    [0, 1, rows - 2, rows - 1]]))
    ti = torch.from_numpy(idx).cuda()
    xs = x[ti].view(torch.int16).cpu().numpy().view(np.uint16)
    gs = g.view(torch.int16).cpu().numpy().view(np.uint16)
    oc, os_, orr = O.mxnorm_fwd(xs, gs, 2, C_DEF[2], O.E4M3)
    P.assert_rho_equal(rho[ti].cpu().numpy(), orr, "tail sampled")
    P.assert_scales_equal(scales[ti].cpu().numpy(), os_, "tail sampled")
    P.assert_codes(codes[ti].cpu().numpy(), oc, os_, O.E4M3, exact=True, what="tail sampled")


def test_mxnorm_default_c_and_optional_rrms():
    xb, gb = W.generate(64, 4096, "outlier", seed=5)
    x, g = P.to_device_bf16(xb), P.to_device_bf16(gb)
    c1, s1, r1 = mxq.mxnorm_fwd(x, g, p=2, c=0.0)
    c2, s2, r2 = mxq.mxnorm_fwd(x, g, p=2, c=0.0, want_rrms=False)
    torch.cuda.synchronize()
    assert r2 is None
    oc, os_, orr = O.mxnorm_fwd(xb, gb, 2, C_DEF[2], 0)
    P.assert_rho_equal(P.from_device(r1), orr)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    P.assert_codes(P.from_device(c1), oc, os_, 0)


@pytest.mark.parametrize("hidden,had", [(2048, 0), (4096, 16), (4096, 32), (8192, 0)])
def test_optional_rrms_every_kernel(hidden, had):
    """Without a rho output every kernel the launcher picks writes the same codes
    and scales."""
    xb, gb = W.generate(37, hidden, "outlier", seed=hidden + had)
    x, g = P.to_device_bf16(xb), P.to_device_bf16(gb)
    if had:
        c1, s1, r1 = mxq.mxnorm_hadamard_fwd(x, g, p=2, c=0.0, had=had, elem=mxq.E2M1)
        c2, s2, r2 = mxq.mxnorm_hadamard_fwd(x, g, p=2, c=0.0, had=had, elem=mxq.E2M1,
                                             want_rrms=False)
    else:
        c1, s1, r1 = mxq.mxnorm_fwd(x, g, p=2, c=0.0)
        c2, s2, r2 = mxq.mxnorm_fwd(x, g, p=2, c=0.0, want_rrms=False)
    torch.cuda.synchronize()
    assert r2 is None and r1 is not None
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


def test_mxnorm_deterministic_and_side_stream():
    xb, gb = W.workload_inputs(2)
    x, g = P.to_device_bf16(xb), P.to_device_bf16(gb)
    a = mxq.mxnorm_fwd(x, g, p=2)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b = mxq.mxnorm_fwd(x, g, p=2, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ------------------------------------------------------------ Hadamard variant

@pytest.mark.parametrize("had", [16, 32])
@pytest.mark.parametrize("elem", [1, 0])
@pytest.mark.parametrize("hidden", [32, 96, 768, 3072, 4096, 5120, 6176, 8192, 10240, 24576])
def test_hadamard_shapes(had, elem, hidden):
    xb, gb = W.generate(41, hidden, "outlier", seed=had + hidden)
    _check_mxnorm(xb, gb, 2, C_DEF[2], elem, had=had, what="H%d D=%d" % (had, hidden))
    _check_mxnorm(xb, None, 1, 1.5, elem, had=had, what="H%d D=%d no gamma" % (had, hidden))


def test_hadamard_workload5_full():
    w = W.WORKLOADS[5]
    xb, gb = W.workload_inputs(5)
    _check_mxnorm(xb, gb, 2, C_DEF[2], w.elem, had=16, what=w.name)


@pytest.mark.parametrize("had", [16, 32])
@pytest.mark.parametrize("elem", [1, 0])
def test_hadamard_edge_rows(had, elem):
    # every rotation kernel at 4096 (a lane per 32-group for E2M1, per 16-group
    # for E4M3 with a gain, one wave per row for H16 -> E4M3 without one)
    xb = _edge_rows(4096)
    gb = _bits(1 + 0.02 * np.random.default_rng(4).standard_normal(4096))
    _check_mxnorm(xb, None, 2, 1.0, elem, had=had, what="H%d elem %d edge" % (had, elem))
    _check_mxnorm(xb, gb, 2, C_DEF[2], elem, had=had, what="H%d elem %d edge gain" % (had, elem))


# ----------------------------------------------------------- two-pass baseline

def _check_baseline(xb, gb, eps, elem, what):
    x = P.to_device_bf16(xb)
    g = None if gb is None else P.to_device_bf16(gb)
    y, codes, scales, rstd = mxq.rmsnorm_mxquant_fwd(x, g, eps=eps, elem=elem)
    torch.cuda.synchronize()
    oy, oc, os_, ors = O.rmsnorm_mxquant_fwd(xb, gb, eps, elem)
    gr = P.from_device(rstd)
    assert np.max(np.abs(gr.astype(np.float64) / ors - 1)) <= 1e-5, what
    gy = P.from_device(y.view(torch.int16)).view(np.uint16)
    dy = np.abs(gy.astype(np.int64) - oy.astype(np.int64))
    assert dy.max() <= 1, what + ": bf16 y differs by more than one ulp"
    gs = P.from_device(scales)
    ds = np.abs(gs.astype(np.int64) - os_.astype(np.int64))
    assert ds.max() <= 1 and np.count_nonzero(ds) <= max(1, 1e-4 * ds.size), what
    P.assert_codes(P.from_device(codes), oc, os_, elem, exact=False, what=what)


def test_baseline_workload2_full():
    xb, gb = W.workload_inputs(2)
    _check_baseline(xb, gb, 1e-5, 0, "two-pass C2")


@pytest.mark.parametrize("hidden", [32, 96, 768, 3104, 4096, 4128, 16384])
@pytest.mark.parametrize("elem", [0, 1])
def test_baseline_shapes(hidden, elem):
    xb, gb = W.generate(33, hidden, "rowscale", seed=hidden + 11)
    _check_baseline(xb, gb, 1e-5, elem, "two-pass D=%d" % hidden)
    _check_baseline(xb, None, 0.0, elem, "two-pass D=%d no gamma" % hidden)


@pytest.mark.parametrize("layout", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("hidden", [2048, 4096])
def test_measure_patterns_move_the_bytes(layout, hidden):
    # every byte-pattern reference reads every input word and writes every
    # output byte of the forward's traffic: check its XOR outputs on the host
    from mx_quantised_tensor_amd import measure
    M = measure.lib()
    if not M.mxq_pattern_supported(layout, hidden):
        pytest.skip("layout %d does not cover hidden %d" % (layout, hidden))
    rows = 37
    rng = np.random.default_rng(99 + layout)
    xw = rng.integers(0, 2 ** 32, size=(rows, hidden // 2), dtype=np.uint32)
    x = torch.from_numpy(xw.view(np.int32)).cuda()
    codes = torch.empty((rows, hidden), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, hidden // 32), dtype=torch.uint8, device="cuda")
    rr = torch.empty((rows,), dtype=torch.float32, device="cuda")
    print("case: pattern layout %d hidden %d" % (layout, hidden), flush=True)
    st = M.mxq_measure_pattern(layout, x.data_ptr(), rows, hidden, codes.data_ptr(),
                               scales.data_ptr(), rr.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    f = np.bitwise_xor.reduce(xw, axis=1)                 # [rows]
    v = xw.reshape(rows, hidden // 8, 4)                  # 16-byte chunks
    lo = v[:, :, 0] ^ v[:, :, 1] ^ f[:, None]
    hi = v[:, :, 2] ^ v[:, :, 3]
    want = np.stack([lo, hi], axis=-1).reshape(rows, -1).view(np.uint8)
    assert np.array_equal(codes.cpu().numpy(), want)
    sw = scales.cpu().numpy().view(np.uint32)
    assert np.array_equal(sw, np.repeat(f[:, None], hidden // 128, axis=1))
    assert np.array_equal(rr.cpu().numpy().view(np.uint32), f)


@pytest.mark.parametrize("waves,hidden", [(2, 4096), (8, 4096), (8, 8192), (2, 1024)])
def test_measure_bwd_pattern_moves_the_bytes(waves, hidden):
    # the backward's byte pattern reads every word of x and dy and writes
    # every word of dx: check its XOR outputs on the host
    from mx_quantised_tensor_amd import measure
    M = measure.lib()
    rows = 37
    rng = np.random.default_rng(7 + waves + hidden)
    xw = rng.integers(0, 2 ** 32, size=(rows, hidden // 2), dtype=np.uint32)
    dw = rng.integers(0, 2 ** 32, size=(rows, hidden // 2), dtype=np.uint32)
    x = torch.from_numpy(xw.view(np.int32)).cuda()
    dy = torch.from_numpy(dw.view(np.int32)).cuda()
    dx = torch.empty_like(x)
    print("case: backward pattern %d waves hidden %d" % (waves, hidden), flush=True)
    st = M.mxq_measure_bwd_pattern(waves, x.data_ptr(), dy.data_ptr(), rows, hidden,
                                   dx.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    f = np.bitwise_xor.reduce(xw, axis=1) ^ np.bitwise_xor.reduce(dw, axis=1)
    assert np.array_equal(dx.cpu().numpy().view(np.uint32), xw ^ dw ^ f[:, None])


def test_mxnorm_maximum_rows_sampled():
    # the largest row count the C ABI accepts (2^24 - 1: the grid then holds
    # 2^22 workgroups), hidden 64, checked on sampled rows that the oracle
    # computes one by one (the first and last rows included)
    rows, hidden = (1 << 24) - 1, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    x = (torch.randn(rows, hidden, device="cuda", generator=gen) * 3.0).to(torch.bfloat16)
    print("case: mxnorm_fwd rows=%d hidden=%d" % (rows, hidden), flush=True)
    codes, scales, rho = mxq.mxnorm_fwd(x, None, p=2, c=C_DEF[2], elem=O.E4M3)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    idx = np.unique(np.concatenate([rng.integers(0, rows, 3000), [0, 1, rows - 2, rows - 1]]))
    ti = torch.from_numpy(idx).cuda()
    xs = x[ti].view(torch.int16).cpu().numpy().view(np.uint16)
    oc, os_, orr = O.mxnorm_fwd(xs, None, 2, C_DEF[2], O.E4M3)
    P.assert_rho_equal(rho[ti].cpu().numpy(), orr, "max rows")
    P.assert_scales_equal(scales[ti].cpu().numpy(), os_, "max rows")
    P.assert_codes(codes[ti].cpu().numpy(), oc, os_, O.E4M3, exact=True, what="max rows")
