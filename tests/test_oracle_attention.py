"""Pins for the oracle's decode attention and bytes-per-token arithmetic.

Attention: on inputs that every format stores losslessly, the oracle over the
packed cache must equal a library attention routine
(torch scaled_dot_product_attention, fp64) on the raw tensors; plus the
special cases single token, identical keys, zero scale, convex hull, ragged
lengths and the query-head -> KV-head grouping.
Bytes: the pages' printed figures, and the byte count of the arrays each
encoder actually produces.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import attention as A
from oracle import e2m1
from oracle import formats as F
from oracle.bytes import bytes_per_token, per_token_head
from oracle.lloyd_max import canonical_codebook
from oracle.numerics import round_bf16
from oracle.rotation import canonical_projection, canonical_rotation


def _sdpa(q, K, V, scale, lens=None):
    """Library attention, fp64: q [B,Hq,dk], K [B,H,T,dk], V [B,H,T,dv] -> [B,Hq,dv]."""
    B, Hq = q.shape[:2]
    H = K.shape[1]
    out = []
    for b in range(B):
        L = K.shape[2] if lens is None else int(lens[b])
        Kb = torch.from_numpy(K[b, :, :L]).repeat_interleave(Hq // H, 0)
        Vb = torch.from_numpy(V[b, :, :L]).repeat_interleave(Hq // H, 0)
        qb = torch.from_numpy(q[b])[:, None, :]
        out.append(Fn.scaled_dot_product_attention(qb, Kb, Vb, scale=scale)[:, 0].numpy())
    return np.stack(out)


def _fp4_grid(rng, shape, top=True):
    """Values stored exactly by FP4: s * E2M1 per 16-channel group, group max = 6 s."""
    *lead, d = shape
    s = round_bf16(np.abs(rng.standard_normal(tuple(lead) + (d // 16,))) * 0.3 + 0.05)
    idx = rng.integers(0, 8, size=tuple(lead) + (d // 16, 16))
    if top:
        idx[..., 0] = 7
    sgn = np.where(rng.integers(0, 2, size=idx.shape), -1.0, 1.0)
    return (sgn * e2m1.MAGNITUDES[idx] * s[..., None]).reshape(shape)


def test_fp4_lossless_equals_library_attention():
    rng = np.random.default_rng(0)
    B, Hq, H, T, d = 2, 8, 2, 96, 32
    K = _fp4_grid(rng, (B, H, T, d))
    V = _fp4_grid(rng, (B, H, T, d))
    q = round_bf16(rng.standard_normal((B, Hq, d)))
    cache = F.encode_cache("fp4", K, V)
    lens = np.array([96, 37])
    got = A.decode_attention("fp4", cache, q, lens, 0.2, H)
    np.testing.assert_allclose(got, _sdpa(q, K, V, 0.2, lens), rtol=0, atol=1e-12)


def test_kivi_lossless_equals_library_attention():
    rng = np.random.default_rng(1)
    B, Hq, H, T, d = 1, 4, 2, 64, 64
    # keys: per (32-token group, channel) grid z + c s; values: per (token, 32-channel group)
    ks = 2.0 ** rng.integers(-2, 2, size=(B, H, T // 32, 1, d))
    kz = rng.integers(-4, 4, size=ks.shape) * 0.25
    kc = rng.integers(0, 4, size=(B, H, T // 32, 32, d))
    kc[..., 0, :], kc[..., 1, :] = 0, 3
    K = (kz + kc * ks).reshape(B, H, T, d)
    vs = 2.0 ** rng.integers(-2, 2, size=(B, H, T, d // 32, 1))
    vz = rng.integers(-4, 4, size=vs.shape) * 0.25
    vc = rng.integers(0, 4, size=(B, H, T, d // 32, 32))
    vc[..., 0], vc[..., 1] = 0, 3
    V = (vz + vc * vs).reshape(B, H, T, d)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32).astype(np.float64)
    cache = F.encode_cache("kivi2", K, V)
    got = A.decode_attention("kivi2", cache, q, [T], 0.125, H)
    np.testing.assert_allclose(got, _sdpa(q, K, V, 0.125), rtol=0, atol=1e-12)


def test_latent_lossless_equals_library_attention():
    rng = np.random.default_rng(2)
    B, Hq, T, dl, dr = 2, 16, 40, 64, 16
    lat = np.concatenate([_fp4_grid(rng, (B, T, dl)), round_bf16(rng.standard_normal((B, T, dr)))], -1)
    q = round_bf16(rng.standard_normal((B, Hq, dl + dr)))
    cache = F.encode_cache("latent", latent=lat, latent_dim=dl)
    got = A.decode_attention("latent", cache, q, [T, 17], 0.1, 1, latent_dim=dl)
    want = _sdpa(q, lat[:, None], lat[:, None, :, :dl], 0.1, [T, 17])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_special_cases_single_identical_zero_scale_hull():
    rng = np.random.default_rng(3)
    B, Hq, H, T, d = 1, 4, 2, 50, 32
    K = round_bf16(rng.standard_normal((B, H, T, d)))
    V = round_bf16(rng.standard_normal((B, H, T, d)))
    q = round_bf16(rng.standard_normal((B, Hq, d)))
    cache = F.encode_cache("fp4", K, V)
    vhat = F.fp4_decode(cache["v_codes"], cache["v_scale"])
    # one token: output is that token's dequantised value, for every head of the group
    one = A.decode_attention("fp4", cache, q, [1], 1.0, H)
    np.testing.assert_allclose(one[0, :2], np.repeat(vhat[0, 0, :1], 2, 0), atol=1e-15)
    np.testing.assert_allclose(one[0, 2:], np.repeat(vhat[0, 1, :1], 2, 0), atol=1e-15)
    # zero scale: the plain mean of the values
    z = A.decode_attention("fp4", cache, q, [T], 0.0, H)
    np.testing.assert_allclose(z[0, 0], vhat[0, 0].mean(0), atol=1e-14)
    # identical keys: also the mean
    K2 = np.repeat(K[:, :, :1], T, 2)
    c2 = F.encode_cache("fp4", K2, V)
    np.testing.assert_allclose(A.decode_attention("fp4", c2, q, [T], 0.7, H)[0, 3],
                               vhat[0, 1].mean(0), atol=1e-14)
    # convex hull: each coordinate between the min and max of the values
    o = A.decode_attention("fp4", cache, q, [T], 3.0, H)
    assert np.all(o[0, :2] <= vhat[0, 0].max(0) + 1e-14) and np.all(o[0, :2] >= vhat[0, 0].min(0) - 1e-14)


def test_group_mapping_and_ragged_tail_ignored():
    rng = np.random.default_rng(4)
    B, Hq, H, T, d = 2, 8, 4, 64, 32
    K = round_bf16(rng.standard_normal((B, H, T, d)))
    V = round_bf16(rng.standard_normal((B, H, T, d)))
    q = round_bf16(rng.standard_normal((B, Hq, d)))
    base = A.decode_attention("fp4", F.encode_cache("fp4", K, V), q, [T, 30], 0.3, H)
    V2 = V.copy()
    V2[:, 1] += 1.0                              # KV head 1 serves query heads 2, 3 only
    V2[1, :, 30:] = 99.0                         # beyond sequence 1's length
    got = A.decode_attention("fp4", F.encode_cache("fp4", K, V2), q, [T, 30], 0.3, H)
    changed = np.any(got != base, axis=-1)
    assert changed.tolist() == [[False, False, True, True, False, False, False, False]] * 2


def test_turbo_and_qjl_rows_api_matches_full():
    rng = np.random.default_rng(5)
    B, Hq, H, T, d = 2, 4, 2, 48, 32
    consts = dict(rot=canonical_rotation(rng.standard_normal((d, d))),
                  proj=canonical_projection(rng.standard_normal((d, d))))
    consts["levels"], consts["thresholds"] = canonical_codebook(2, d)
    K = round_bf16(rng.standard_normal((B, H, T, d)))
    V = round_bf16(rng.standard_normal((B, H, T, d)))
    q = round_bf16(rng.standard_normal((B, Hq, d)))
    for fmt in ("turbo", "qjl1"):
        cache = F.encode_cache(fmt, K, V, consts=consts)
        full = A.decode_attention(fmt, cache, q, [T, 20], 0.2, H, consts)
        rows = A.decode_attention(fmt, cache, q, [T, 20], 0.2, H, consts, rows=[(1, 3), (0, 0)])
        np.testing.assert_allclose(rows[(1, 3)], full[1, 3], rtol=0, atol=1e-13)
        np.testing.assert_allclose(rows[(0, 0)], full[0, 0], rtol=0, atol=1e-13)


# ----------------------------------------------------------------- bytes

def test_bytes_per_token_printed_figures(golden):
    for layers, heads, d, tokens, want, _ in golden("bytes_per_token.txt"):
        got = bytes_per_token("bf16", int(heads), int(d), int(layers)) * int(tokens)
        assert got == int(want)
    assert abs(bytes_per_token("bf16", 8, 128, 80) / 2 ** 20 - 0.31) < 0.005


@pytest.mark.parametrize("fmt,d,rope", [("fp4", 128, 0), ("kivi2", 64, 0), ("kivi2", 128, 0),
                                        ("turbo", 128, 0), ("qjl1", 128, 0), ("latent", 512, 64)])
def test_bytes_per_token_equals_encoded_arrays(fmt, d, rope):
    rng = np.random.default_rng(6)
    T = 64
    consts = dict(rot=canonical_rotation(rng.standard_normal((d, d))),
                  proj=canonical_projection(rng.standard_normal((128, d))))
    consts["levels"], consts["thresholds"] = canonical_codebook(2, d)
    if fmt == "latent":
        lat = round_bf16(rng.standard_normal((1, T, d + rope)))
        enc = F.encode_cache(fmt, latent=lat, latent_dim=d)
        per = sum(a.nbytes for a in enc.values()) / T
    else:
        K = round_bf16(rng.standard_normal((1, 1, T, d)))
        enc = F.encode_cache(fmt, K, K.copy(), consts=consts)
        per = sum(a.nbytes for a in enc.values()) / T
    assert per == per_token_head(fmt, d, rope)
    assert {"fp4": 160, "turbo": 86, "qjl1": 98, "latent": 448}.get(fmt, d) == per
