"""E2M1 (FP4) element encoding.

The pages store the main KV cache as FP4 E2M1 (OCP MX element format) with one
scale per 16 channels (page "How DeepSeek-V4.1-Flash cut KV-cache storage by 4x
via CSA2", section on numerical precision and hardware efficiency; page
"DeepSeek-V4.1-Flash cuts KV cache to 890 bytes per token", spec list).

An E2M1 nibble is s e1 e0 m: sign, two exponent bits (bias 1), one mantissa
bit.  Exponent 0 is subnormal (0 or 0.5); magnitudes, in code order 0..7:
    0, 0.5, 1, 1.5, 2, 3, 4, 6
Reading taken for encoding (the pages name the format only): the magnitude
index is the one whose value times the scale is nearest |x| in exact
arithmetic; an exact tie goes to the even index (mantissa bit 0); anything
beyond 6*s saturates to 6; the sign bit is the sign bit of x, so -0.0 and a
negative value that rounds to 0 both encode 0x8.
"""

import numpy as np

MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def magnitude_index(absx, s):
    """Nearest E2M1 magnitude index of absx / s, ties to even index.

    absx, s: fp64 arrays (broadcastable), s > 0.  Compares |absx - s*m_i| over
    all eight magnitudes; s*m_i is exact in fp64 for bf16 s, so the distance
    comparison decides ties exactly.
    """
    absx = np.asarray(absx, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    cand = s[..., None] * MAGNITUDES                    # [..., 8]
    dist = np.abs(absx[..., None] - cand)
    best = np.argmin(dist, axis=-1)                      # first (lowest) index on ties
    # an exact tie between neighbours i and i+1: argmin picked i; move to the even one
    dmin = np.take_along_axis(dist, best[..., None], -1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    tie = (nxt != best) & (np.take_along_axis(dist, nxt[..., None], -1)[..., 0] == dmin)
    best = np.where(tie & (best % 2 == 1), nxt, best)
    return best.astype(np.uint8)


def encode(x, s):
    """Nibble (uint8 0..15) of x with scale s; s == 0 encodes 0."""
    x = np.asarray(x, dtype=np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), x.shape)
    idx = magnitude_index(np.abs(x), np.where(s > 0, s, 1.0))
    sign = np.signbit(x).astype(np.uint8)
    nib = (sign << 3) | idx
    return np.where(s > 0, nib, 0).astype(np.uint8)


def decode(nib):
    """fp64 value of nibbles (no scale)."""
    nib = np.asarray(nib, dtype=np.uint8)
    mag = MAGNITUDES[nib & 7]
    return np.where(nib & 8, -mag, mag)
