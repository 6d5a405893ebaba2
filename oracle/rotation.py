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
