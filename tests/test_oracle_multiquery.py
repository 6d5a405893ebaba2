"""Pins for the oracle's several-queries-per-sequence decode (causal tail mask).

- On inputs FP4 stores losslessly, the oracle equals a library attention
  routine (torch scaled_dot_product_attention, fp64) given the mask that lets
  query j of nq see the first L - (nq - 1 - j) tokens.
- One query per sequence reduces to the single-query oracle.
- Query j alone is the single-query oracle over L - (nq - 1 - j) tokens, for
  every format (this catches a mask off by one or aligned to the wrong end).
- With L = nq the first query sees one token: its output is that token's value.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import attention as A
from oracle import e2m1
from oracle import formats as F
from oracle.lloyd_max import canonical_codebook
from oracle.numerics import round_bf16
from oracle.rotation import canonical_projection, canonical_rotation


def _fp4_grid(rng, shape):
    *lead, d = shape
    s = round_bf16(np.abs(rng.standard_normal(tuple(lead) + (d // 16,))) * 0.3 + 0.05)
    idx = rng.integers(0, 8, size=tuple(lead) + (d // 16, 16))
    idx[..., 0] = 7
    sgn = np.where(rng.integers(0, 2, size=idx.shape), -1.0, 1.0)
    return (sgn * e2m1.MAGNITUDES[idx] * s[..., None]).reshape(shape)


def test_fp4_lossless_equals_library_masked_attention():
    rng = np.random.default_rng(10)
    B, nq, Hq, H, T, d = 2, 5, 8, 2, 70, 32
    K = _fp4_grid(rng, (B, H, T, d))
    V = _fp4_grid(rng, (B, H, T, d))
    q = round_bf16(rng.standard_normal((B, nq, Hq, d)))
    lens = np.array([70, 9])
    got = A.decode_attention_multi("fp4", F.encode_cache("fp4", K, V), q, lens, 0.25, H)
    for b in range(B):
        L = int(lens[b])
        mask = torch.zeros(nq, L, dtype=torch.bool)
        for j in range(nq):
            mask[j, :L - (nq - 1 - j)] = True
        Kb = torch.from_numpy(K[b, :, :L]).repeat_interleave(Hq // H, 0)      # [Hq, L, d]
        Vb = torch.from_numpy(V[b, :, :L]).repeat_interleave(Hq // H, 0)
        qb = torch.from_numpy(np.ascontiguousarray(q[b].transpose(1, 0, 2)))  # [Hq, nq, d]
        want = Fn.scaled_dot_product_attention(qb, Kb, Vb, attn_mask=mask, scale=0.25).numpy()
        np.testing.assert_allclose(got[b], want.transpose(1, 0, 2), rtol=0, atol=1e-12)


def _caches(rng):
    B, H, T, d = 2, 2, 64, 32
    consts = dict(rot=canonical_rotation(rng.standard_normal((d, d))),
                  proj=canonical_projection(rng.standard_normal((d, d))))
    consts["levels"], consts["thresholds"] = canonical_codebook(2, d)
    K = round_bf16(rng.standard_normal((B, H, T, d)))
    V = round_bf16(rng.standard_normal((B, H, T, d)))
    out = {f: (F.encode_cache(f, K, V, consts=consts), d, 512) for f in ("fp4", "turbo", "qjl1")}
    kv = round_bf16(rng.standard_normal((B, H, T, 64)))
    out["kivi2"] = (F.encode_cache("kivi2", kv, kv), 64, 512)
    lat = np.concatenate([_fp4_grid(rng, (B, T, 64)), round_bf16(rng.standard_normal((B, T, 16)))], -1)
    out["latent"] = (F.encode_cache("latent", latent=lat, latent_dim=64), 80, 64)
    return out, consts


@pytest.mark.parametrize("fmt", ["fp4", "turbo", "qjl1", "kivi2", "latent"])
def test_each_query_is_the_single_query_decode_over_its_prefix(fmt):
    rng = np.random.default_rng(11)
    caches, consts = _caches(rng)
    cache, dk, dl = caches[fmt]
    H = 1 if fmt == "latent" else 2
    B, nq, Hq = 2, 4, 4
    q = round_bf16(rng.standard_normal((B, nq, Hq, dk)))
    lens = np.array([64, 6])
    multi = A.decode_attention_multi(fmt, cache, q, lens, 0.3, H, consts, latent_dim=dl)
    for j in range(nq):
        single = A.decode_attention(fmt, cache, q[:, j], lens - (nq - 1 - j), 0.3, H, consts, latent_dim=dl)
        np.testing.assert_allclose(multi[:, j], single, rtol=0, atol=1e-12)
    one = A.decode_attention_multi(fmt, cache, q[:, :1], lens, 0.3, H, consts, latent_dim=dl)
    np.testing.assert_allclose(one[:, 0], A.decode_attention(fmt, cache, q[:, 0], lens, 0.3, H, consts,
                                                             latent_dim=dl), rtol=0, atol=1e-12)


def test_first_query_over_nq_tokens_sees_one_token():
    rng = np.random.default_rng(12)
    B, nq, Hq, H, T, d = 1, 3, 2, 1, 3, 32
    K = round_bf16(rng.standard_normal((B, H, T, d)))
    V = round_bf16(rng.standard_normal((B, H, T, d)))
    cache = F.encode_cache("fp4", K, V)
    vhat = F.fp4_decode(cache["v_codes"], cache["v_scale"])
    q = round_bf16(rng.standard_normal((B, nq, Hq, d)))
    out = A.decode_attention_multi("fp4", cache, q, [T], 5.0, H)
    np.testing.assert_allclose(out[0, 0], np.repeat(vhat[0, 0, :1], Hq, 0), atol=1e-15)
    with pytest.raises(ValueError):
        A.decode_attention_multi("fp4", cache, q, [2], 1.0, H)
