"""Round-to-nearest-even into narrow floating formats, in fp64 arithmetic.

A value is split as m * 2**e with m in [0.5, 1) (numpy.frexp); keeping p
significant bits means rounding m * 2**p to an integer, ties to even
(numpy.rint), then scaling back.  Below the format's smallest normal the
spacing is fixed at the subnormal step.  Overflow goes to +-inf (fp16) or
+-inf past bf16's largest finite value.
"""

import numpy as np


def _round_sig(x, p: int, emin: int, max_finite: float):
    """RNE of fp64 array x to p significant bits, normal exponent >= emin."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    m, e = np.frexp(x[nz])               # x = m * 2**e, 0.5 <= |m| < 1
    # value = (m * 2**p) * 2**(e - p); normal numbers have e - 1 >= emin
    shift = np.maximum(e, emin + 1) - p  # exponent of one unit in the last place
    q = np.rint(np.ldexp(x[nz], -shift))
    r = np.ldexp(q, shift)
    r = np.where(np.abs(r) > max_finite, np.copysign(np.inf, r), r)
    out[nz] = r
    # keep the sign of zero
    out[~nz] = x[~nz]
    return out


def round_bf16(x):
    """bf16: 8 significant bits, min normal 2**-126, max finite (2 - 2**-7) * 2**127."""
    return _round_sig(x, 8, -126, float(np.ldexp(2.0 - 2.0 ** -7, 127)))


def round_fp16(x):
    """fp16: 11 significant bits, min normal 2**-14, max finite 65504."""
    return _round_sig(x, 11, -14, 65504.0)


def round_fp32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16-representable fp64 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def fp16_bits(x) -> np.ndarray:
    """uint16 bit patterns of fp16-representable fp64 values."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_from_bits(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)
