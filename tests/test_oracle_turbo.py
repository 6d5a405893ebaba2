"""Pins for the oracle's rotation, QJL sketch and TurboQuant estimator.

* Haar rotation: orthogonality, the sign convention of the QR factor, and the
  distribution of a rotated unit vector's coordinates (N(0, 1/d)).
* QJL: the logit estimate is unbiased over the draw of S, with the closed-form
  variance ((pi/2) |q|^2 |r|^2 - <q,r>^2) / m (the Gaussian identity behind the
  1-bit JL transform).
* TurboQuant: the distortion of the rotated Lloyd-Max stage stays within the
  stated ~2.7x of the 4^-b lower bound, and the full estimator is unbiased over S.
"""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import formats as F
from oracle.lloyd_max import canonical_codebook
from oracle.numerics import fp16_from_bits, round_bf16
from oracle.rotation import canonical_projection, canonical_rotation, haar_rotation


def _gauss(seed, r, c):
    return np.random.default_rng(seed).standard_normal((r, c))


def test_haar_orthogonal_and_sign_convention():
    g = _gauss(0, 128, 128)
    q = haar_rotation(g)
    np.testing.assert_allclose(q.T @ q, np.eye(128), atol=1e-12)
    r = q.T @ g                                   # must be the upper-triangular factor
    assert np.max(np.abs(np.tril(r, -1))) < 1e-10
    assert np.all(np.diag(r) > 0)
    assert abs(abs(np.linalg.det(q)) - 1) < 1e-10
    rc = canonical_rotation(g)
    np.testing.assert_array_equal(rc, round_bf16(rc))
    assert np.max(np.abs(rc.T @ rc - np.eye(128))) < 4e-3


def test_haar_rotated_coordinates_are_gaussian():
    d, n = 32, 3000
    x = np.zeros(d)
    x[0] = 1.0
    coords = np.array([haar_rotation(_gauss(s, d, d)) @ x for s in range(n)])
    var = coords.var()
    assert abs(var - 1.0 / d) < 0.1 / d
    kurt = np.mean(coords ** 4) / np.mean(coords ** 2) ** 2
    assert abs(kurt - 3.0 * d / (d + 2)) < 0.25       # a uniform-sphere coordinate: 3d/(d+2)
    np.testing.assert_allclose((coords ** 2).sum(1), 1.0, atol=1e-12)


def test_qjl_unbiased_with_closed_form_variance():
    d, m, n = 64, 64, 20000
    rng = np.random.default_rng(5)
    q = rng.standard_normal(d)
    r = rng.standard_normal(d) * 0.3
    kap = A.qjl_kappa(m)
    est = np.empty(n)
    for s in range(n):
        S = _gauss(10_000 + s, m, d)
        est[s] = kap * np.linalg.norm(r) * (S @ q) @ np.where(S @ r >= 0, 1.0, -1.0)
    truth = q @ r
    var_cf = ((math.pi / 2) * (q @ q) * (r @ r) - truth ** 2) / m
    se = math.sqrt(var_cf / n)
    assert abs(est.mean() - truth) < 4 * se
    assert abs(est.var() / var_cf - 1) < 0.05


def test_qjl_cache_logit_unbiased_through_encoder():
    """The same estimate taken through the oracle's encoder and decode logit path."""
    d, m, n = 32, 32, 4000
    rng = np.random.default_rng(6)
    k = round_bf16(rng.standard_normal(d))
    q = rng.standard_normal(d)
    ests = np.empty(n)
    for s in range(n):
        S = canonical_projection(_gauss(50_000 + s, m, d))
        cache = {kk: v[None, None, None] for kk, v in F.qjl_encode_keys(k, S).items()}
        ests[s] = A._key_logits("qjl1", cache, 0, 0, 0, 1, q[None], {"proj": S}, 0)[0, 0]
    n_k = fp16_from_bits(F.norms_fp16(k))
    truth = q @ k * n_k / np.linalg.norm(k)
    var_cf = ((math.pi / 2) * (q @ q) * (k @ k) - (q @ k) ** 2) / m
    assert abs(ests.mean() - truth) < 4 * math.sqrt(var_cf / n)


@pytest.mark.parametrize("bits,bound", [(1, 2.7 / 4), (2, 2.7 / 16)])
def test_turbo_distortion_within_bound(bits, bound):
    d, n = 128, 4000
    rot = haar_rotation(_gauss(1, d, d))
    levels, thr = canonical_codebook(bits, d)
    x = _gauss(2, n, d)
    _, u, idx = F.turbo_stage1(x, rot, levels, thr)
    mse = np.mean(((u - levels[idx]) ** 2).sum(-1))
    assert mse <= bound
    # and close to the Gaussian Lloyd-Max distortion per coordinate times d
    ref = {1: 1 - 2 / math.pi, 2: 0.11748}[bits]
    assert abs(mse - ref) < 0.02


def test_turbo_residual_identity_and_unbiased_logit():
    """<q,k> = n (<Rq, u_tilde> + <Rq, r>); the sketch term estimates the second part without bias."""
    d, m, n = 64, 64, 3000
    rot = haar_rotation(_gauss(3, d, d))
    levels, thr = canonical_codebook(2, d)
    rng = np.random.default_rng(7)
    k = round_bf16(rng.standard_normal(d) * 2)
    q = round_bf16(rng.standard_normal(d))
    nk, u, idx = F.turbo_stage1(k, rot, levels, thr)
    r = u - levels[idx]
    assert abs(nk * ((rot @ q) @ levels[idx] + (rot @ q) @ r) - q @ k) < 1e-10
    ests = np.empty(n)
    for s in range(n):
        S = canonical_projection(_gauss(90_000 + s, m, d))
        enc = F.turbo_encode_keys(k, rot, S, levels, thr)
        cache = {kk: v[None, None, None] for kk, v in enc.items()}
        consts = dict(rot=rot, proj=S, levels=levels, thresholds=thr)
        ests[s] = A._key_logits("turbo", cache, 0, 0, 0, 1, q[None], consts, 0)[0, 0]
    n16 = fp16_from_bits(F.norms_fp16(k))
    g16 = fp16_from_bits(F.turbo_encode_keys(k, rot, S, levels, thr)["k_rnorm"])
    truth = n16 * ((rot @ q) @ levels[idx] + (rot @ q) @ r * g16 / np.linalg.norm(r))
    spread = n16 * g16 * math.sqrt(math.pi / 2 * (q @ q) / m)
    assert abs(ests.mean() - truth) < 4 * spread / math.sqrt(n)


def test_turbo_decode_fidelity_single_token_and_logits():
    """Value path: one token's output is n_v R^T u_tilde, within the stage-one distortion of v
    (a transposed or missing R would give an error near sqrt(2)).  Logit path: estimates
    track the exact <q, k> over many tokens."""
    d, m, T = 128, 128, 4096
    rot = canonical_rotation(_gauss(11, d, d))
    S = canonical_projection(_gauss(12, m, d))
    levels, thr = canonical_codebook(2, d)
    consts = dict(rot=rot, proj=S, levels=levels, thresholds=thr)
    rng = np.random.default_rng(13)
    K = round_bf16(rng.standard_normal((1, 1, T, d)))
    V = round_bf16(rng.standard_normal((1, 1, T, d)))
    q = round_bf16(rng.standard_normal((1, 1, d)))
    cache = F.encode_cache("turbo", K, V, consts=consts)
    for t in range(8):
        sub = {k: v[:, :, t:t + 1] for k, v in cache.items()}
        o = A.decode_attention("turbo", sub, q, [1], 1.0, 1, consts)[0, 0]
        rel = np.linalg.norm(o - V[0, 0, t]) / np.linalg.norm(V[0, 0, t])
        assert rel < 0.45, rel
    est = A._key_logits("turbo", cache, 0, 0, 0, T, q[0], consts, 0)[0]
    exact = K[0, 0] @ q[0, 0]
    err = est - exact
    assert abs(np.mean(err)) < 4 * np.std(err) / math.sqrt(T)
    # error variance near the QJL closed form (averaged over S; one S here, so loosely)
    nk, u, idx = F.turbo_stage1(K[0, 0], rot, levels, thr)
    r = u - levels[idx]
    qr = rot @ q[0, 0]
    pred = nk ** 2 * ((math.pi / 2) * (qr @ qr) * (r * r).sum(-1) - (r @ qr) ** 2) / m
    assert 0.6 < np.mean(err ** 2) / np.mean(pred) < 1.4
    assert np.corrcoef(est, exact)[0, 1] > 0.85
