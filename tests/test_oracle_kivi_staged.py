"""Pins for the oracle's KIVI-2 decode with the last incomplete key group read
from the input keys.

- Whole groups only (L a multiple of 32), or a prefix of a longer append whose
  groups are all coded: the plain oracle.
- Everything staged (L < 32): a library attention routine (torch
  scaled_dot_product_attention, fp64) on the input keys and the values the
  oracle's KIVI value decoder gives.
- Which keys are read: changing the packed key codes of the staged tokens, or
  the input keys of tokens in whole groups, leaves the output unchanged; the
  input key of a staged token does not.
"""

import numpy as np
import torch
import torch.nn.functional as Fn

from oracle import attention as A
from oracle import formats as F


def _setup(rng, B=2, H=2, T=96, d=64):
    K = rng.standard_normal((B, H, T, d)).astype(np.float32).astype(np.float64)
    V = rng.standard_normal((B, H, T, d)).astype(np.float32).astype(np.float64)
    return K, V, F.encode_cache("kivi2", K, V)


def test_whole_groups_are_the_plain_oracle():
    rng = np.random.default_rng(30)
    K, V, cache = _setup(rng)
    q = rng.standard_normal((2, 2, 4, 64))
    lens = np.array([96, 64])
    np.testing.assert_allclose(A.decode_attention_kivi_staged(cache, q, lens, 0.2, 2, K),
                               A.decode_attention_multi("kivi2", cache, q, lens, 0.2, 2), rtol=0, atol=1e-12)


def test_all_staged_is_library_attention_on_input_keys():
    rng = np.random.default_rng(31)
    K, V, cache = _setup(rng)
    q = rng.standard_normal((2, 1, 4, 64))
    lens = np.array([29, 5])
    got = A.decode_attention_kivi_staged(cache, q, lens, 0.3, 2, K)
    vhat = F.kivi2_decode_values(cache["v_codes"], cache["v_scale"], cache["v_zero"])
    for b in range(2):
        L = int(lens[b])
        Kb = torch.from_numpy(K[b, :, :L]).repeat_interleave(2, 0)
        Vb = torch.from_numpy(vhat[b, :, :L]).repeat_interleave(2, 0)
        want = Fn.scaled_dot_product_attention(torch.from_numpy(q[b, 0])[:, None], Kb, Vb, scale=0.3)[:, 0].numpy()
        np.testing.assert_allclose(got[b, 0], want, rtol=0, atol=1e-12)


def test_each_key_comes_from_its_own_representation():
    rng = np.random.default_rng(32)
    K, V, cache = _setup(rng, B=1)
    q = rng.standard_normal((1, 1, 4, 64))
    L = 75                                           # groups 0, 1 whole; tokens 64..74 staged
    base = A.decode_attention_kivi_staged(cache, q, [L], 0.4, 2, K)
    c2 = {k: v.copy() for k, v in cache.items()}
    c2["k_codes"][:, :, 64:] ^= 0x55
    np.testing.assert_array_equal(A.decode_attention_kivi_staged(c2, q, [L], 0.4, 2, K), base)
    K2 = K.copy()
    K2[:, :, :64] += 3.0
    np.testing.assert_array_equal(A.decode_attention_kivi_staged(cache, q, [L], 0.4, 2, K2), base)
    for t in (64, 74):
        K3 = K.copy()
        K3[:, :, t] += 1.0
        assert not np.array_equal(A.decode_attention_kivi_staged(cache, q, [L], 0.4, 2, K3), base)
    K4 = K.copy()
    K4[:, :, 63] += 1.0                              # last token of a whole group: read packed
    np.testing.assert_array_equal(A.decode_attention_kivi_staged(cache, q, [L], 0.4, 2, K4), base)


def test_prefix_of_a_longer_append_reads_coded_groups():
    rng = np.random.default_rng(33)
    K, V, cache = _setup(rng)
    q = rng.standard_normal((2, 1, 4, 64))
    lens, appended = np.array([40, 7]), np.array([96, 40])
    np.testing.assert_allclose(A.decode_attention_kivi_staged(cache, q, lens, 0.2, 2, K, appended),
                               A.decode_attention_multi("kivi2", cache, q, lens, 0.2, 2), rtol=0, atol=1e-12)
    # the same prefix of a sequence appended only that far stages its last group
    assert not np.allclose(A.decode_attention_kivi_staged(cache, q, lens, 0.2, 2, K, lens),
                           A.decode_attention_multi("kivi2", cache, q, lens, 0.2, 2))
