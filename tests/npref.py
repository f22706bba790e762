"""Independent numpy restatements used to pin the oracle (tests only).

These take a different route from the oracle's C code on purpose: element
rounding uses numpy's round-half-to-even on a per-binade integer grid (the
oracle searches a table of all codes), and floor(log2) uses numpy's log2 (the
oracle uses frexp).  A mistake in either route shows up as a disagreement.
"""
import numpy as np

E4M3, E2M1 = 0, 1
# (mantissa bits, smallest normal exponent, largest finite value, emax)
FMT = {E4M3: (3, -6, 448.0, 8), E2M1: (1, 0, 6.0, 2)}


def bf16_bits_to_f64(b):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(b).astype(np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def f32_to_bf16_bits(f):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def round_elem(v, elem):
    """Nearest element value (ties to even), saturating; returns float64."""
    mbits, emin, vmax, _ = FMT[elem]
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        eb = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    eb = np.maximum(eb, emin)
    step = np.exp2(eb - mbits)
    q = np.minimum(np.round(a / step) * step, vmax)
    return np.copysign(q, v)


def floor_log2(a):
    with np.errstate(divide="ignore"):
        return np.floor(np.log2(a))


def scale_exp(amax, elem):
    """E8M0 exponent for a block absmax (float64 array); 128 marks NaN."""
    emax = FMT[elem][3]
    amax = np.asarray(amax, dtype=np.float64)
    fin = np.isfinite(amax)
    safe = np.where(fin & (amax > 0), amax, 1.0)
    e = floor_log2(safe) - emax
    e = np.where(amax == 0, -127, e)
    e = np.clip(e, -127, 127)
    return np.where(fin, e, 128).astype(np.int64)


def quantise_blocks(y, elem):
    """MX cast of a float64 matrix [rows, hidden] (values already final).

    Returns (values [rows, hidden] float64 = decoded codes, scale exponents
    [rows, K] int64 with 128 = NaN scale)."""
    rows, hidden = y.shape
    b = y.reshape(rows, hidden // 32, 32)
    fin = np.all(np.isfinite(b), axis=2)
    amax = np.where(fin, np.max(np.abs(np.where(np.isfinite(b), b, 0.0)), axis=2), np.inf)
    e = scale_exp(amax, elem)
    eb = np.where(e == 128, 0, e)[:, :, None].astype(np.float64)
    q = round_elem(b / np.exp2(eb), elem)
    return q.reshape(rows, hidden), e


def decode_codes(codes, elem, hidden):
    """Oracle/GPU codes -> float64 element values (not scaled)."""
    import oracle as O  # decode tables are pinned separately against torch
    if elem == E4M3:
        tab = np.array([O.e4m3_decode(c) for c in range(256)])
        return tab[codes]
    tab = np.array([O.e2m1_decode(c) for c in range(16)])
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty(codes.shape[:-1] + (hidden,), dtype=np.float64)
    out[..., 0::2] = tab[lo]
    out[..., 1::2] = tab[hi]
    return out


def code_signs(codes, elem, hidden):
    if elem == E4M3:
        return (codes >> 7).astype(bool)
    out = np.empty(codes.shape[:-1] + (hidden,), dtype=bool)
    out[..., 0::2] = (codes >> 3) & 1
    out[..., 1::2] = (codes >> 7) & 1
    return out
