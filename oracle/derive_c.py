"""Default correction constant c(p, B) of the MXNorm estimator -- derivation.

The estimator scales the power mean of the block magnitudes by c(p, B); the
summary of the MXNorm paper (P1, "Resumen técnico" §2, "Fundamentos
Teóricos" / "Fórmula") says the constant is precalculated and depends on the
block size and the input distribution, but prints no value.  This script
derives it for i.i.d. Gaussian activations, block size B = 32, and block
magnitudes taken from the E8M0 scales (a power of two, 2^floor(log2 absmax)).

Let M be the max of B i.i.d. |N(0,1)|.  Its p-th moment is
    E[M^p] = integral_0^inf p m^(p-1) (1 - erf(m / sqrt 2)^B) dm.
With the row scale sigma log-uniform, the fractional binary exponent f of
sigma*M is uniform on [0, 1), so the power-of-two magnitude 2^-f sigma M has
    E[mt^p] = sigma^p E[M^p] (1 - 2^-p) / (p ln 2),
and c = (E[M^p] (1 - 2^-p) / (p ln 2))^(1/p) makes c * E[mt^p]^(-1/p) equal to
1/sigma = 1/RMS.  Output (B = 32): c(1) ~ 1.69306, c(2) ~ 1.75753.
"""
import math

from scipy import integrate, special


def moment_of_block_max(p: int, B: int = 32) -> float:
    f = lambda m: p * m ** (p - 1) * (1.0 - special.erf(m / math.sqrt(2.0)) ** B)
    val, _ = integrate.quad(f, 0.0, math.inf, limit=200, epsabs=1e-13, epsrel=1e-13)
    return val


def c_exact_absmax(p: int, B: int = 32) -> float:
    """Constant for the exact block absmax (not used by the library)."""
    return moment_of_block_max(p, B) ** (1.0 / p)


def c_pow2_scale(p: int, B: int = 32) -> float:
    """Constant for power-of-two block magnitudes (the E8M0-scale reading)."""
    m = moment_of_block_max(p, B)
    return (m * (1.0 - 2.0 ** (-p)) / (p * math.log(2.0))) ** (1.0 / p)


if __name__ == "__main__":
    import numpy as np
    for p in (1, 2):
        c = c_pow2_scale(p)
        print("p=%d  E[M^p]=%.7f  c_exact=%.7f  c_pow2=%.7f  (fp32 %s)" % (
            p, moment_of_block_max(p), c_exact_absmax(p), c,
            hex(np.float32(c).view(np.uint32))))
