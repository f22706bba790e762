"""Seeded synthetic activations for the MXNorm workloads.

This module only draws random inputs; it holds none of the method's
arithmetic and is shared, unchanged, by the GPU tests, the CPU oracle tests
and the benchmark.  bf16 rounding of the drawn fp32 values uses torch's
round-to-nearest-even conversion (a library routine).

The pages time the norm on Llama 3 layer activations (1B: hidden 2048,
8B: hidden 4096) but print neither data nor shapes; these generators stand in
for them with the shapes and value structure of the five workloads:

  * x ~ N(0, 1) in fp32, then 1% of the hidden channels (the same channels in
    every row, drawn without replacement) multiplied by 20 -- the outlier
    channels of LLM activations;
  * gamma = 1 + 0.02 * N(0, 1) per channel (an RMSNorm gain), bf16;
  * "rowscale": each row times exp(N(0, 1)), a log-normal (sigma = 1) row scale;
  * "t3": 0.1% of all entries, drawn without replacement, replaced by
    50 * Student-t(3) samples (heavy-tailed, exercises saturation);
  * finally x is rounded to bf16.

Draw order is fixed (x, outlier channels, gamma, then the per-workload extra)
so a workload is a pure function of (seed, rows, hidden, kind).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

E4M3 = 0
E2M1 = 1


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    hidden: int
    ps: Tuple[int, ...]
    elem: int
    had: int            # 0 = no rotation, 16 = H16
    kind: str           # "outlier", "rowscale" or "t3"
    seed: int
    two_pass: bool = False
    notes: str = field(default="", compare=False)


WORKLOADS = {
    1: Workload("mxnorm_p2_e4m3_256x768", 256, 768, (2,), E4M3, 0, "outlier", 1,
                notes="small case the CPU oracle finishes in seconds"),
    2: Workload("mxnorm_p1p2_e4m3_8192x2048", 8192, 2048, (1, 2), E4M3, 0, "outlier", 2,
                two_pass=True, notes="Llama-3 1B shape; p=1 and p=2 vs the two-pass baseline"),
    3: Workload("mxnorm_p2_e4m3_16384x4096", 16384, 4096, (2,), E4M3, 0, "rowscale", 3,
                notes="Llama-3 8B shape (4 x 4096 tokens); the headline workload"),
    4: Workload("mxnorm_p2_e2m1_16384x4096", 16384, 4096, (2,), E2M1, 0, "t3", 4,
                notes="MXFP4 elements with heavy-tailed entries"),
    5: Workload("mxnorm_h16_p2_e2m1_32768x4096", 32768, 4096, (2,), E2M1, 16, "outlier", 5,
                notes="deterministic H16 rotation then MXFP4"),
}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even (torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def generate(rows: int, hidden: int, kind: str, seed: int,
             row_subset: Optional[slice] = None):
    """Return (x_bits [rows, hidden] uint16, gamma_bits [hidden] uint16).

    ``row_subset`` keeps only those rows of the full draw (the draw itself is
    unchanged, so a subset is exactly the same data as in the full matrix).
    """
    if hidden % 32 != 0:
        raise ValueError("hidden must be a multiple of 32")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, hidden), dtype=np.float32)
    n_out = int(round(0.01 * hidden))
    if n_out > 0:
        ch = rng.choice(hidden, n_out, replace=False)
        x[:, ch] *= np.float32(20.0)
    gamma = (1.0 + 0.02 * rng.standard_normal(hidden)).astype(np.float32)
    if kind == "rowscale":
        x *= np.exp(rng.standard_normal((rows, 1))).astype(np.float32)
    elif kind == "t3":
        n = int(round(0.001 * rows * hidden))
        if n > 0:
            pos = rng.choice(rows * hidden, n, replace=False)
            x.reshape(-1)[pos] = (50.0 * rng.standard_t(3, n)).astype(np.float32)
    elif kind != "outlier":
        raise ValueError("unknown workload kind %r" % kind)
    if row_subset is not None:
        x = x[row_subset]
    return to_bf16_bits(x), to_bf16_bits(gamma)


def grad_output(rows: int, hidden: int, seed: int, scale: float = 1.0):
    """Incoming gradient for the backward: scale * N(0, 1), bf16 bits.  Drawn
    from its own stream (seed + 7919), so it does not disturb the forward draw."""
    rng = np.random.default_rng(seed + 7919)
    dy = rng.standard_normal((rows, hidden), dtype=np.float32)
    return to_bf16_bits(dy * np.float32(scale))


def workload_inputs(cfg: int, row_subset: Optional[slice] = None):
    w = WORKLOADS[cfg]
    return generate(w.rows, w.hidden, w.kind, w.seed, row_subset)


def random_rows(rows: int, hidden: int, seed: int, scale_spread: float = 0.0):
    """Plain Gaussian rows for small tests: N(0,1) times an optional per-row
    log-uniform scale 2^U(-spread/2, spread/2)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, hidden), dtype=np.float32)
    if scale_spread:
        u = rng.uniform(-scale_spread / 2, scale_spread / 2, size=(rows, 1))
        x *= np.exp2(u).astype(np.float32)
    return x


def linear_weight(out_features: int, hidden: int, seed: int):
    """Weight of the linear layer after the norm: N(0, 1/hidden) (fan-in
    scaling), bf16 bits, [out_features, hidden].  Own stream (seed + 104729)."""
    rng = np.random.default_rng(seed + 104729)
    w = rng.standard_normal((out_features, hidden), dtype=np.float32)
    return to_bf16_bits(w * np.float32(1.0 / np.sqrt(hidden)))
