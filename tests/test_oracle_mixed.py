"""Pins for the oracle's mixed-precision decode (bf16 sink and recent tokens,
packed history), for FP4-valued, KIVI-2 and TurboQuant histories.

- No window: the plain (multi-query) oracle (KIVI-2: the staged oracle).
- A window that covers the whole context: a library attention routine (torch
  scaled_dot_product_attention, fp64) on the bf16 inputs, with the causal tail
  mask for several queries.
- Which representation each token uses: changing the packed codes of window
  tokens, or the inputs of history tokens, leaves the output unchanged, while
  changing a window token's input does not.
- TurboQuant: a window over a history whose packed part is lossless in the
  rotated basis (every token a codebook point times a norm) equals library
  attention on the dequantised history and the bf16 window, so the window's
  values enter in the original basis and the history's through R^T.
- KIVI-2 with an incomplete key group and a recent window shorter than it: the
  staged tokens outside the window attend with their exact keys, those inside
  with bf16 keys (library attention on keys assembled token by token).
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import attention as A
from oracle import formats as F
from oracle.numerics import round_bf16
from oracle.lloyd_max import canonical_codebook
from oracle.rotation import canonical_projection, canonical_rotation

FMTS = ["fp4", "qjl1", "kivi2", "turbo"]


def _setup(fmt, rng, B=2, H=2, T=96, d=32):
    if fmt == "turbo":
        d = 128                                              # TurboQuant's codebook is for d = 128
    K = round_bf16(rng.standard_normal((B, H, T, d)))
    V = round_bf16(rng.standard_normal((B, H, T, d)))
    consts = None
    if fmt == "qjl1":
        consts = dict(proj=canonical_projection(rng.standard_normal((d, d))))
    if fmt == "turbo":
        lv, th = canonical_codebook(2, d)
        consts = dict(rot=canonical_rotation(rng.standard_normal((d, d))),
                      proj=canonical_projection(rng.standard_normal((d, d))), levels=lv, thresholds=th)
    return K, V, consts, F.encode_cache(fmt, K, V, consts=consts)


@pytest.mark.parametrize("fmt", FMTS)
def test_no_window_is_the_plain_oracle(fmt):
    rng = np.random.default_rng(20)
    K, V, consts, cache = _setup(fmt, rng)
    d = K.shape[-1]
    q = round_bf16(rng.standard_normal((2, 3, 4, d)))
    lens = np.array([96, 64]) if fmt == "kivi2" else np.array([80, 41])   # whole KIVI groups: nothing staged
    got = A.decode_attention_mixed(fmt, cache, q, lens, 0.3, 2, K, V, 0, 0, consts)
    want = A.decode_attention_multi(fmt, cache, q, lens, 0.3, 2, consts)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_no_window_kivi_staged_is_the_staged_oracle():
    rng = np.random.default_rng(25)
    K, V, consts, cache = _setup("kivi2", rng)
    q = round_bf16(rng.standard_normal((2, 2, 4, 32)))
    lens = np.array([80, 41])
    got = A.decode_attention_mixed("kivi2", cache, q, lens, 0.3, 2, K, V, 0, 0)
    want = A.decode_attention_kivi_staged(cache, q, lens, 0.3, 2, K)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fmt", FMTS)
def test_full_window_is_library_attention_on_bf16(fmt):
    rng = np.random.default_rng(21)
    K, V, consts, cache = _setup(fmt, rng)
    B, nq, Hq, H = 2, 3, 4, 2
    q = round_bf16(rng.standard_normal((B, nq, Hq, K.shape[-1])))
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


@pytest.mark.parametrize("fmt", FMTS)
def test_each_token_uses_its_own_representation(fmt):
    rng = np.random.default_rng(22)
    K, V, consts, cache = _setup(fmt, rng, B=1, T=64)
    q = round_bf16(rng.standard_normal((1, 1, 4, K.shape[-1])))
    S, W, L = 5, 9, 64
    mixed = lambda c, k, v: A.decode_attention_mixed(fmt, c, q, [L], 0.5, 2, k, v, S, W, consts)
    base = mixed(cache, K, V)
    # packed codes of window tokens are not read
    c2 = {k: v.copy() for k, v in cache.items()}
    for t in list(range(S)) + list(range(L - W, L)):
        for name in c2:
            if c2[name].ndim == 4 and name.endswith("codes"):   # per-token code rows
                c2[name][:, :, t] ^= 0x11
    np.testing.assert_array_equal(mixed(c2, K, V), base)
    # inputs of history tokens are not read
    K2, V2 = K.copy(), V.copy()
    K2[:, :, S:L - W] += 1.0
    V2[:, :, S:L - W] -= 1.0
    np.testing.assert_array_equal(mixed(cache, K2, V2), base)
    # a window token's input is
    for t in (0, S - 1, L - W, L - 1):
        V3 = V.copy()
        V3[:, :, t] += 0.5
        assert not np.array_equal(mixed(cache, K, V3), base)
    # the first token past the sink and the last before the recent window are read packed
    for t in (S, L - W - 1):
        V4 = V.copy()
        V4[:, :, t] += 0.5
        np.testing.assert_array_equal(mixed(cache, K, V4), base)


def _sdpa(q, Kb, Vb, scale):
    """Library attention (torch, fp64): q [Hq, d], Kb / Vb [H, L, d]."""
    Hq, H = q.shape[0], Kb.shape[0]
    Kr = torch.from_numpy(np.ascontiguousarray(Kb)).repeat_interleave(Hq // H, 0)
    Vr = torch.from_numpy(np.ascontiguousarray(Vb)).repeat_interleave(Hq // H, 0)
    qt = torch.from_numpy(np.ascontiguousarray(q))[:, None, :]
    return Fn.scaled_dot_product_attention(qt, Kr, Vr, scale=scale)[:, 0].numpy()


def test_turbo_window_is_library_attention_in_the_original_basis():
    """TurboQuant history values are stored in the rotated basis; the window's bf16
    values are in the original one.  The softmax over estimator logits (history) and
    bf16 dot products (window) is taken by library attention with the history's
    logits as an additive mask over zero keys; the history's values must come back
    to the original basis through R^T, which the second half checks against the
    inputs themselves: 2-bit Lloyd-Max keeps about 88% of a unit vector's energy,
    so the decoded history lies within 0.5 of the input, relative, in the right
    basis and about sqrt(2) away in the rotated one (or through R instead of R^T)."""
    rng = np.random.default_rng(23)
    d, H, L, S, W = 128, 1, 48, 4, 6
    K, V, consts, cache = _setup("turbo", rng, B=1, H=H, T=L)
    rot = np.asarray(consts["rot"], np.float64)
    win = np.zeros(L, bool)
    win[:S] = win[L - W:] = True
    q = round_bf16(rng.standard_normal((1, 1, 2, d)))
    got = A.decode_attention_mixed("turbo", cache, q, [L], 0.2, H, K, V, S, W, consts)[0, 0]
    stored = A._values("turbo", cache, 0, 0, 0, L, consts, 0)          # rotated basis
    hist = stored @ rot                                                 # R^T applied to each row
    est = A._key_logits("turbo", cache, 0, 0, 0, L, q[0, 0], consts, 0)
    keys = np.where(win[:, None], round_bf16(K[0, 0]), 0.0)[None]
    bias = np.where(win[None, :], 0.0, est * 0.2)                       # [Hq, L]
    vals = np.where(win[:, None], round_bf16(V[0, 0]), hist)[None]
    qt = torch.from_numpy(np.ascontiguousarray(q[0, 0]))[:, None, :]
    want = Fn.scaled_dot_product_attention(
        qt, torch.from_numpy(keys).expand(2, L, d), torch.from_numpy(vals).expand(2, L, d),
        attn_mask=torch.from_numpy(bias)[:, None, :], scale=0.2)[:, 0].numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    v = V[0, 0][~win]
    rel = lambda x: np.linalg.norm(x - v, axis=1) / np.linalg.norm(v, axis=1)
    assert rel(hist[~win]).max() < 0.5
    assert rel(stored[~win]).min() > 1.0
    assert rel((stored @ rot.T)[~win]).min() > 1.0


def test_kivi_staged_keys_outside_the_window_are_exact():
    rng = np.random.default_rng(24)
    H, T, d = 2, 96, 32
    K = rng.standard_normal((1, H, T, d))                     # fp32-exact keys: bf16 rounding changes them
    K = K.astype(np.float32).astype(np.float64)
    V = rng.standard_normal((1, H, T, d)).astype(np.float32).astype(np.float64)
    cache = F.encode_cache("kivi2", K, V)
    L, S, W = 70, 0, 4                                        # tokens 64..69 staged, 66..69 in the window
    q = round_bf16(rng.standard_normal((1, 1, 4, d)))
    got = A.decode_attention_mixed("kivi2", cache, q, [L], 0.4, H, K, V, S, W)[0, 0]
    # keys assembled token by token: coded groups, exact staged keys, bf16 window keys
    kc = np.stack([F.kivi2_decode_keys(cache["k_codes"][0, h, :64], cache["k_scale"][0, h, :2],
                                       cache["k_zero"][0, h, :2]) for h in range(H)])
    Kb = np.concatenate([kc, K[0, :, 64:66], round_bf16(K[0, :, 66:70])], axis=1)
    vc = np.stack([F.kivi2_decode_values(cache["v_codes"][0, h, :66], cache["v_scale"][0, h, :66],
                                         cache["v_zero"][0, h, :66]) for h in range(H)])
    Vb = np.concatenate([vc, round_bf16(V[0, :, 66:70])], axis=1)
    np.testing.assert_allclose(got, _sdpa(q[0, 0], Kb, Vb, 0.4), rtol=0, atol=1e-12)
    # the staged tokens outside the window really are read exact (bf16 would differ)
    Kb2 = Kb.copy()
    Kb2[:, 64:66] = round_bf16(K[0, :, 64:66])
    assert np.abs(_sdpa(q[0, 0], Kb2, Vb, 0.4) - got).max() > 1e-9
