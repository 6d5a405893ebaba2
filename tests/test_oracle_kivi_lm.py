"""Pins for the oracle's KIVI 2-bit coding and the Gaussian Lloyd-Max quantiser."""

import math

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

from oracle import formats as F
from oracle.lloyd_max import canonical_codebook, gaussian_lloyd_max, quantize_index


# ----------------------------------------------------------------- KIVI

def test_kivi_lossless_grid_keys_and_values():
    rng = np.random.default_rng(0)
    # z + c*s with s a power of two and z on a coarse grid: all fp32 steps exact
    s = 2.0 ** rng.integers(-3, 3, size=(2, 64))          # per (token group, channel)
    z = rng.integers(-8, 8, size=(2, 64)) * 0.125
    c = rng.integers(0, 4, size=(2, 32, 64))
    c[:, 0, :], c[:, 1, :] = 0, 3                            # min and max present in every group
    k = (z[:, None, :] + c * s[:, None, :]).reshape(64, 64)
    codes, ks, kz = F.kivi2_encode_keys(k)
    np.testing.assert_array_equal(F.unpack_2bit(codes), c.reshape(64, 64))
    np.testing.assert_array_equal(ks, s.astype(np.float32))
    np.testing.assert_array_equal(kz, z.astype(np.float32))
    np.testing.assert_array_equal(F.kivi2_decode_keys(codes, ks, kz), k)
    # values: the same grid laid out per token over 32-channel groups
    v = k.T.copy()                                           # now channels x ... ; regroup per token
    vc, vs, vz = F.kivi2_encode_values(v)
    np.testing.assert_array_equal(F.kivi2_decode_values(vc, vs, vz), v)


def test_kivi_axes_keys_per_channel_values_per_token():
    """An outlier channel changes only its own key scale; an outlier token only its own value groups."""
    rng = np.random.default_rng(1)
    k = rng.standard_normal((64, 64)).astype(np.float32).astype(np.float64)
    base_c, base_s, _ = F.kivi2_encode_keys(k)
    k2 = k.copy()
    k2[:, 5] *= 20.0
    c2, s2, _ = F.kivi2_encode_keys(k2)
    changed = np.nonzero(np.any(s2 != base_s, axis=0))[0]
    assert changed.tolist() == [5]
    v = rng.standard_normal((64, 64)).astype(np.float32).astype(np.float64)
    _, vs, _ = F.kivi2_encode_values(v)
    v2 = v.copy()
    v2[7, :] *= 20.0
    _, vs2, _ = F.kivi2_encode_values(v2)
    assert np.nonzero(np.any(vs2 != vs, axis=1))[0].tolist() == [7]


def test_kivi_constant_group_min_max_and_nearest():
    k = np.ones((32, 8)) * 0.7
    codes, s, z = F.kivi2_encode_keys(k)
    assert np.all(F.unpack_2bit(codes) == 0) and np.all(s == 0)
    np.testing.assert_array_equal(F.kivi2_decode_keys(codes, s, z), np.float32(0.7).astype(np.float64) * np.ones((32, 8)))
    rng = np.random.default_rng(2)
    x = rng.standard_normal((32 * 8, 16)).astype(np.float32).astype(np.float64)
    codes, s, z = F.kivi2_encode_keys(x)
    c = F.unpack_2bit(codes).reshape(8, 32, 16)
    g = x.reshape(8, 32, 16)
    assert np.all(c[np.arange(8)[:, None], g.argmin(1), np.arange(16)[None]] == 0)
    assert np.all(c[np.arange(8)[:, None], g.argmax(1), np.arange(16)[None]] == 3)
    # nearest level in exact arithmetic, except within fp32 rounding of a midpoint
    levels = z[:, None, None, :] + np.arange(4)[None, None, :, None] * s[:, None, None, :]
    d = np.abs(g[:, :, None, :] - levels)
    best = d.argmin(2)
    mid = (g - z[:, None, :]) / s[:, None, :] - 0.5
    near_tie = np.abs(mid - np.round(mid)) < 1e-5
    assert np.all((best == c) | near_tie)


# ----------------------------------------------------------------- Lloyd-Max

def test_lloyd_max_against_published_table(golden):
    for bits, kind, i, val in golden("lloyd_max_gaussian.txt"):
        bits, i, val = int(bits), int(i), float(val)
        lv, th = gaussian_lloyd_max(bits)
        if kind == "mse":
            got = _mse(lv, th)
        elif kind == "level":
            got = lv[i]
        else:
            got = th[i]
        tol = 1e-9 if bits == 1 else 6e-4 * max(1.0, abs(val))
        assert abs(got - val) <= tol, (bits, kind, i, got, val)


def _mse(lv, th):
    edges = np.concatenate(([-np.inf], th, [np.inf]))
    tot = 0.0
    for j, c in enumerate(lv):
        tot += integrate.quad(lambda z: (z - c) ** 2 * norm.pdf(z), edges[j], edges[j + 1],
                              epsabs=1e-13, epsrel=1e-12)[0]
    return tot


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_lloyd_max_optimality_by_quadrature(bits):
    lv, th = gaussian_lloyd_max(bits)
    np.testing.assert_allclose(th, 0.5 * (lv[:-1] + lv[1:]), atol=1e-14)
    edges = np.concatenate(([-np.inf], th, [np.inf]))
    for j, c in enumerate(lv):
        mass = integrate.quad(norm.pdf, edges[j], edges[j + 1], epsabs=1e-14)[0]
        mean = integrate.quad(lambda z: z * norm.pdf(z), edges[j], edges[j + 1], epsabs=1e-14)[0] / mass
        assert abs(mean - c) < 1e-9
    assert np.all(np.diff(lv) > 0)
    np.testing.assert_array_equal(lv, -lv[::-1])          # symmetric source, symmetric optimum
    assert th[len(th) // 2] == 0.0


def test_lloyd_max_sigma_scaling_and_canonical():
    lv1, th1 = gaussian_lloyd_max(2, 1.0)
    lv, th = gaussian_lloyd_max(2, 0.25)
    np.testing.assert_allclose(lv, 0.25 * lv1, rtol=1e-15)
    clv, cth = canonical_codebook(2, 128)
    np.testing.assert_array_equal(clv, (lv1 / math.sqrt(128)).astype(np.float32))
    np.testing.assert_array_equal(cth, (th1 / math.sqrt(128)).astype(np.float32))


def test_quantize_index_tie_selects_upper_cell():
    th = np.array([-0.5, 0.0, 0.5])
    assert quantize_index(np.array([-1.0, -0.5, -0.1, 0.0, 0.49, 0.5, 2.0]), th).tolist() == [0, 1, 1, 2, 2, 3, 3]
