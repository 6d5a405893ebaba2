"""Pins for the oracle's structured rotation (Hadamard transform with a
bit-reversal permutation, the OSCAR paragraph of the TurboQuant vs OSCAR page,
section "quantization frontiers: TurboQuant and OSCAR").

* The Sylvester recursion agrees with the closed form H[i, j] = (-1)^popcount(i & j)
  and H H^T = d I.
* The permutation is the bit reversal of FFT index order: the order of 8 is
  0 4 2 6 1 5 3 7, it is an involution, and rev(2^k) = d / 2^(k+1).
* R x equals a fast Walsh-Hadamard butterfly of the permuted x over sqrt(d), so
  R's orientation (R[i, j] multiplies x[j]) and the side the permutation acts on
  are fixed.
* The stored bf16 matrix has every entry +-bf16(1/sqrt(d)) and R R^T = a^2 d I
  exactly; a one-hot channel is spread evenly over every output coordinate.
* With 2-bit Lloyd-Max codes the distortion of unit vectors stays within ~2.7x of
  the 4^-b lower bound, on Gaussian keys and on keys with a few outlier channels
  where the identity rotation exceeds it.
"""

import math

import numpy as np
import pytest

from oracle import formats as F
from oracle.lloyd_max import canonical_codebook
from oracle.numerics import round_bf16
from oracle.rotation import bit_reversal, canonical_hadamard_rotation, hadamard_rotation, sylvester_hadamard

DIMS = [1, 2, 4, 8, 16, 32, 64, 128, 256]


@pytest.mark.parametrize("d", DIMS)
def test_sylvester_closed_form_and_orthogonality(d):
    h = sylvester_hadamard(d)
    want = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
    np.testing.assert_array_equal(h, want)
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


def test_bit_reversal_order():
    assert list(bit_reversal(8)) == [0, 4, 2, 6, 1, 5, 3, 7]
    assert list(bit_reversal(2)) == [0, 1]
    for d in DIMS:
        rev = bit_reversal(d)
        assert sorted(rev) == list(range(d))
        np.testing.assert_array_equal(rev[rev], np.arange(d))
        for k in range(d.bit_length() - 1):
            assert rev[1 << k] == d >> (k + 1)
    with pytest.raises(ValueError):
        bit_reversal(12)


def _fwht(x):
    """In-place butterfly: pairs (i, i + h) -> (a + b, a - b) for h = 1, 2, 4, ..."""
    y = np.array(x, dtype=np.float64)
    h = 1
    while h < y.shape[-1]:
        for i in range(0, y.shape[-1], 2 * h):
            a = y[..., i:i + h].copy()
            b = y[..., i + h:i + 2 * h].copy()
            y[..., i:i + h] = a + b
            y[..., i + h:i + 2 * h] = a - b
        h *= 2
    return y


@pytest.mark.parametrize("d", [8, 64, 128])
def test_rotation_is_butterfly_of_permuted_input(d):
    x = np.random.default_rng(d).standard_normal((5, d))
    rev = bit_reversal(d)
    np.testing.assert_allclose(x @ hadamard_rotation(d).T, _fwht(x[:, rev]) / math.sqrt(d), atol=1e-12)
    np.testing.assert_allclose(x @ hadamard_rotation(d, bit_reverse=False).T, _fwht(x) / math.sqrt(d),
                               atol=1e-12)
    # permutation first: for d = 8 the input channel 1 meets Walsh column 4
    if d == 8:
        e1 = np.eye(8)[1]
        np.testing.assert_allclose(hadamard_rotation(8) @ e1 * math.sqrt(8), [1, 1, 1, 1, -1, -1, -1, -1])


@pytest.mark.parametrize("d", [16, 64, 128])
def test_stored_matrix_is_scaled_orthogonal(d):
    r = canonical_hadamard_rotation(d)
    a = round_bf16(np.array([1 / math.sqrt(d)]))[0]
    np.testing.assert_array_equal(np.abs(r), np.full((d, d), a))
    np.testing.assert_array_equal(r @ r.T, (a * a * d) * np.eye(d))
    assert abs(a * a * d - 1) < 2 ** -8
    # a single loud channel lands on every coordinate with the same magnitude
    for j in (0, 3, d - 1):
        np.testing.assert_array_equal(np.abs(r @ np.eye(d)[j]), np.full(d, a))


def _unit_distortion(x, rot, bits):
    levels, thr = canonical_codebook(bits, x.shape[-1])
    _, u, idx = F.turbo_stage1(x, rot, levels, thr)
    return np.mean(((u - levels[idx]) ** 2).sum(-1))


def test_distortion_within_bound_and_outliers_spread():
    d, n, bound = 128, 3000, 2.7 / 16
    rng = np.random.default_rng(11)
    x = rng.standard_normal((n, d))
    had = canonical_hadamard_rotation(d)
    g = _unit_distortion(x, had, 2)
    assert g <= bound and abs(g - 0.11748) < 0.02
    xo = x.copy()
    xo[:, [5, 6, 40, 99]] *= 20.0              # a few loud channels, the case the page names
    assert _unit_distortion(xo, had, 2) <= bound
    assert _unit_distortion(xo, np.eye(d), 2) > bound
