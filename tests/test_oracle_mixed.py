"""Pins for the oracle's mixed-precision decode (bf16 sink and recent tokens,
packed history).

- No window: the plain (multi-query) oracle.
- A window that covers the whole context: a library attention routine (torch
  scaled_dot_product_attention, fp64) on the bf16 inputs, with the causal tail
  mask for several queries.
- Which representation each token uses: changing the packed codes of window
  tokens, or the inputs of history tokens, leaves the output unchanged, while
  changing a window token's input does not.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import attention as A
from oracle import formats as F
from oracle.numerics import round_bf16
from oracle.rotation import canonical_projection


def _setup(fmt, rng, B=2, H=2, T=80, d=32):
    K = round_bf16(rng.standard_normal((B, H, T, d)))
    V = round_bf16(rng.standard_normal((B, H, T, d)))
    consts = None
    if fmt == "qjl1":
        consts = dict(proj=canonical_projection(rng.standard_normal((d, d))))
    return K, V, consts, F.encode_cache(fmt, K, V, consts=consts)


@pytest.mark.parametrize("fmt", ["fp4", "qjl1"])
def test_no_window_is_the_plain_oracle(fmt):
    rng = np.random.default_rng(20)
    K, V, consts, cache = _setup(fmt, rng)
    q = round_bf16(rng.standard_normal((2, 3, 4, 32)))
    lens = np.array([80, 41])
    got = A.decode_attention_mixed(fmt, cache, q, lens, 0.3, 2, K, V, 0, 0, consts)
    want = A.decode_attention_multi(fmt, cache, q, lens, 0.3, 2, consts)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fmt", ["fp4", "qjl1"])
def test_full_window_is_library_attention_on_bf16(fmt):
    rng = np.random.default_rng(21)
    K, V, consts, cache = _setup(fmt, rng)
    B, nq, Hq, H = 2, 3, 4, 2
    q = round_bf16(rng.standard_normal((B, nq, Hq, 32)))
    lens = np.array([80, 41])
    got = A.decode_attention_mixed(fmt, cache, q, lens, 0.3, H, K, V, 16, 70, consts)
    for b in range(B):
        L = int(lens[b])
        mask = torch.zeros(nq, L, dtype=torch.bool)
        for j in range(nq):
            mask[j, :L - (nq - 1 - j)] = True
        Kb = torch.from_numpy(K[b, :, :L]).repeat_interleave(Hq // H, 0)
        Vb = torch.from_numpy(V[b, :, :L]).repeat_interleave(Hq // H, 0)
        qb = torch.from_numpy(np.ascontiguousarray(q[b].transpose(1, 0, 2)))
        want = Fn.scaled_dot_product_attention(qb, Kb, Vb, attn_mask=mask, scale=0.3).numpy()
        np.testing.assert_allclose(got[b], want.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_each_token_uses_its_own_representation():
    rng = np.random.default_rng(22)
    K, V, consts, cache = _setup("fp4", rng, B=1, T=64)
    q = round_bf16(rng.standard_normal((1, 1, 4, 32)))
    S, W, L = 5, 9, 64
    base = A.decode_attention_mixed("fp4", cache, q, [L], 0.5, 2, K, V, S, W)
    # packed codes of window tokens are not read
    c2 = {k: v.copy() for k, v in cache.items()}
    for t in list(range(S)) + list(range(L - W, L)):
        c2["k_codes"][:, :, t] ^= 0x11
        c2["v_codes"][:, :, t] ^= 0x22
    np.testing.assert_array_equal(A.decode_attention_mixed("fp4", c2, q, [L], 0.5, 2, K, V, S, W), base)
    # inputs of history tokens are not read
    K2, V2 = K.copy(), V.copy()
    K2[:, :, S:L - W] += 1.0
    V2[:, :, S:L - W] -= 1.0
    np.testing.assert_array_equal(A.decode_attention_mixed("fp4", cache, q, [L], 0.5, 2, K2, V2, S, W), base)
    # a window token's input is
    for t in (0, S - 1, L - W, L - 1):
        V3 = V.copy()
        V3[:, :, t] += 0.5
        assert not np.array_equal(A.decode_attention_mixed("fp4", cache, q, [L], 0.5, 2, K, V3, S, W), base)
    # the first token past the sink and the last before the recent window are read packed
    for t in (S, L - W - 1):
        V4 = V.copy()
        V4[:, :, t] += 0.5
        np.testing.assert_array_equal(A.decode_attention_mixed("fp4", cache, q, [L], 0.5, 2, K, V4, S, W), base)
