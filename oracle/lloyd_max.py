"""Lloyd-Max scalar quantiser for a Gaussian source.

TurboQuant's first stage rotates each vector at random so that its coordinates
are close to independent Gaussians, then applies a precomputed optimal scalar
(Lloyd-Max) quantiser per coordinate (page "TurboQuant vs OSCAR vs EpiCache:
the battle over KV-cache compression", section "quantization frontiers:
TurboQuant and OSCAR", stage one).

Reading taken: the source is N(0, sigma^2) with sigma^2 = 1/d (a unit vector's
coordinates after a random rotation), b bits give 2**b levels, and the
quantiser is the fixed point of the two Lloyd conditions, iterated in fp64:
  * each threshold is the midpoint of its two neighbouring levels;
  * each level is the mean of the source over its cell:
      E[Z | a < Z < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a))  (standard normal).
Levels are returned in ascending order, thresholds likewise; index i codes the
cell [t_{i-1}, t_i) with t_{-1} = -inf, t_{2^b-1} = +inf.
"""

import math

import numpy as np
from scipy.special import ndtr


def _phi(z):
    return np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def gaussian_lloyd_max(bits: int, sigma: float = 1.0, iters: int = 100000, tol: float = 1e-15):
    """(levels[2**bits], thresholds[2**bits - 1]) in fp64 for N(0, sigma^2)."""
    n = 1 << bits
    # start from evenly spread levels over +-2 sigma (standard units)
    lv = np.linspace(-2.0, 2.0, n) if n > 1 else np.zeros(1)
    for _ in range(iters):
        th = 0.5 * (lv[:-1] + lv[1:])
        a = np.concatenate(([-np.inf], th))
        b = np.concatenate((th, [np.inf]))
        pa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
        pb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
        mass = ndtr(b) - ndtr(a)
        new = (pa - pb) / mass
        # the source is symmetric about 0, so is the optimum: keep the iterate
        # exactly antisymmetric (rounding would otherwise leave the middle
        # threshold a few 1e-18 off zero)
        new = 0.5 * (new - new[::-1])
        done = np.max(np.abs(new - lv)) <= tol
        lv = new
        if done:
            break
    th = 0.5 * (lv[:-1] + lv[1:])
    return lv * sigma, th * sigma


def canonical_codebook(bits: int, dim: int):
    """fp32-rounded (levels, thresholds) for N(0, 1/dim), as fp64 arrays."""
    lv, th = gaussian_lloyd_max(bits, 1.0)
    s = 1.0 / math.sqrt(dim)
    return (lv * s).astype(np.float32).astype(np.float64), (th * s).astype(np.float32).astype(np.float64)


def quantize_index(u, thresholds):
    """Cell index of each u: the number of thresholds t with t <= u (a tie selects the upper cell)."""
    u = np.asarray(u, dtype=np.float64)
    return (u[..., None] >= np.asarray(thresholds, dtype=np.float64)).sum(-1).astype(np.uint8)
