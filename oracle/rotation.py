"""Random rotation and QJL projection matrices.

TurboQuant rotates every vector by a random orthogonal matrix before scalar
quantisation, and sketches the residual with a 1-bit quantised
Johnson-Lindenstrauss transform (page "TurboQuant vs OSCAR vs EpiCache: the
battle over KV-cache compression", section "quantization frontiers: TurboQuant
and OSCAR").

Readings taken (the pages name the steps only):
  * the rotation is Haar-distributed: Q from the QR factorisation of a d x d
    matrix of iid N(0,1) draws, with each column of Q multiplied by the sign of
    the matching diagonal entry of R, so that the factorisation is the unique
    one with a positive diagonal;
  * both matrices are stored as bf16-representable values (rounded to nearest
    even once), so that a bf16 matrix-core product with bf16 inputs is exact
    per term;
  * rot[i][j] multiplies x[j]: y = rot @ x.  The inverse used on decode is the
    transpose of the stored (rounded) matrix.
"""

import numpy as np

from .numerics import round_bf16


def haar_rotation(gauss: np.ndarray) -> np.ndarray:
    """fp64 orthogonal Q from the sign-fixed QR of a square Gaussian matrix."""
    q, r = np.linalg.qr(np.asarray(gauss, dtype=np.float64))
    sgn = np.sign(np.diag(r))
    sgn[sgn == 0] = 1.0
    return q * sgn[None, :]


def canonical_rotation(gauss: np.ndarray) -> np.ndarray:
    return round_bf16(haar_rotation(gauss))


def canonical_projection(gauss: np.ndarray) -> np.ndarray:
    """QJL matrix S (m x d): iid N(0,1) draws rounded to bf16."""
    return round_bf16(np.asarray(gauss, dtype=np.float64))


# ---------------------------------------------------------------- structured rotation
#
# The OSCAR paragraph of the same page (section "quantization frontiers:
# TurboQuant and OSCAR") replaces a random rotation by a Hadamard transform
# combined with a bit-reversal permutation, so that a few large channels are
# spread evenly over the quantisation groups.  Readings taken (the page names
# the two ingredients only):
#   * H is the Sylvester Hadamard matrix of order d (d a power of two), built by
#     the recursion H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]], scaled by
#     1/sqrt(d) so that the rotation is orthogonal;
#   * the permutation acts first: y = H (P x) / sqrt(d) with (P x)_i = x_rev(i),
#     rev(i) the index whose log2(d)-bit binary digits are those of i reversed;
#   * the result is stored, like the random rotation, as bf16 values (every
#     entry is +-1/sqrt(d), one bf16 number up to sign), so R R^T = c^2 I with
#     c = bf16(1/sqrt(d)) sqrt(d) close to 1; the decode inverse stays R^T.


def bit_reversal(d: int) -> np.ndarray:
    """rev(i) for i < d, d a power of two: the binary digits of i read backwards."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    nbits = d.bit_length() - 1
    rev = np.zeros(d, dtype=np.int64)
    for i in range(d):
        r = 0
        for b in range(nbits):
            if i >> b & 1:
                r |= 1 << (nbits - 1 - b)
        rev[i] = r
    return rev


def sylvester_hadamard(d: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix of order d by doubling."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_rotation(d: int, bit_reverse: bool = True) -> np.ndarray:
    """fp64 R = H P / sqrt(d): R[i, j] multiplies x[j], so column j of R is column
    rev(j) of H (P is its own inverse)."""
    h = sylvester_hadamard(d)
    if bit_reverse:
        h = h[:, bit_reversal(d)]
    return h / np.sqrt(d)


def canonical_hadamard_rotation(d: int, bit_reverse: bool = True) -> np.ndarray:
    return round_bf16(hadamard_rotation(d, bit_reverse))
