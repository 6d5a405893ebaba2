"""Pins for the oracle's HSI selection and sparse decode.

* Candidate pool: a hand-worked example with ties and a ragged last block;
  positions at or past L never count; all blocks are kept when fewer exist than
  asked for; on random inputs the pool is a union of whole (clipped) blocks,
  their number is min(top_blocks, blocks), and no kept block loses to a dropped
  one (a larger maximum, or an equal one at a lower index).
* Top-k: a hand-worked example with ties; on random pools the same exchange
  property, ascending output, and the size min(k, pool).
* Sparse decode: over every position it is the dense decode; over one position
  it is that position's value; over any selection it is the dense decode of a
  cache holding only the selected tokens.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import formats as F
from oracle.hsi import block_maxima, candidate_pool, decode_attention_sparse, select_top_k


def test_pool_worked_example():
    # L = 21: blocks [0,8) [8,16) [16,21); maxima 5, 7, 5 (ties: block 0 before 2)
    s = np.zeros(32, np.float32)
    s[3], s[9], s[17] = 5, 7, 5
    s[25] = 100.0                                  # past L: ignored
    assert list(candidate_pool(s, 21, 8, 1)) == list(range(8, 16))
    assert list(candidate_pool(s, 21, 8, 2)) == list(range(0, 16))
    assert list(candidate_pool(s, 21, 8, 3)) == list(range(21))
    assert list(candidate_pool(s, 21, 8, 9)) == list(range(21))
    s[20] = 6.0                                    # the clipped last block now beats block 0
    assert list(candidate_pool(s, 21, 8, 2)) == list(range(8, 21))
    assert candidate_pool(s, 0, 8, 4).size == 0
    # -0 and +0 are equal scores: the lower block wins
    z = np.array([-0.0] * 4 + [0.0] * 4, np.float32)
    assert list(candidate_pool(z, 8, 4, 1)) == [0, 1, 2, 3]


@pytest.mark.parametrize("seed,L,block,top", [(0, 1000, 8, 20), (1, 4096, 8, 100), (2, 77, 8, 3),
                                               (3, 5000, 4, 2000), (4, 3000, 8, 10000)])
def test_pool_properties(seed, L, block, top):
    rng = np.random.default_rng(seed)
    s = np.round(rng.standard_normal(L + 50) * 4).astype(np.float32)   # many ties
    pool = candidate_pool(s, L, block, top)
    nb = -(-L // block)
    m = block_maxima(s, L, block)
    kept = sorted(set((pool // block).tolist()))
    assert len(kept) == min(top, nb)
    expect = [t for j in kept for t in range(j * block, min(L, (j + 1) * block))]
    assert pool.tolist() == expect and np.all(np.diff(pool) > 0)
    dropped = sorted(set(range(nb)) - set(kept))
    if dropped:
        worst_kept = min(kept, key=lambda j: (m[j], -j))
        best_dropped = max(dropped, key=lambda j: (m[j], -j))
        assert m[worst_kept] > m[best_dropped] or (m[worst_kept] == m[best_dropped] and worst_kept < best_dropped)


def test_select_worked_example():
    pool = np.array([3, 4, 9, 10, 11, 40], np.int32)
    sc = np.array([1.0, 2.0, 2.0, -1.0, 2.0, 0.5], np.float32)
    assert select_top_k(pool, sc, 1).tolist() == [4]
    assert select_top_k(pool, sc, 2).tolist() == [4, 9]
    assert select_top_k(pool, sc, 4).tolist() == [3, 4, 9, 11]
    assert select_top_k(pool, sc, 99).tolist() == pool.tolist()


@pytest.mark.parametrize("seed,n,k", [(0, 300, 50), (1, 16384, 512), (2, 10, 512)])
def test_select_properties(seed, n, k):
    rng = np.random.default_rng(seed)
    pool = np.sort(rng.choice(100000, n, replace=False)).astype(np.int32)
    sc = np.round(rng.standard_normal(n) * 8).astype(np.float32)
    sel = select_top_k(pool, sc, k)
    assert sel.size == min(k, n) and np.all(np.diff(sel) > 0)
    idx = np.searchsorted(pool, sel)
    mask = np.zeros(n, bool)
    mask[idx] = True
    if (~mask).any():
        kept, dropped = np.flatnonzero(mask), np.flatnonzero(~mask)
        wk = min(kept, key=lambda i: (sc[i], -i))
        bd = max(dropped, key=lambda i: (sc[i], -i))
        assert sc[wk] > sc[bd] or (sc[wk] == sc[bd] and wk < bd)


def _fp4_cache(rng, B, H, T, d):
    K = rng.standard_normal((B, H, T, d))
    V = rng.standard_normal((B, H, T, d))
    return F.encode_cache("fp4", K, V)


def test_sparse_decode_reduces_to_dense_and_compact_cache():
    rng = np.random.default_rng(5)
    B, H, T, d, G = 2, 2, 90, 64, 3
    enc = _fp4_cache(rng, B, H, T, d)
    q = rng.standard_normal((B, H * G, d))
    full = [np.arange(T), np.arange(T)]
    np.testing.assert_allclose(decode_attention_sparse("fp4", enc, q, full, 0.2, H),
                               A.decode_attention("fp4", enc, q, [T, T], 0.2, H), rtol=1e-12, atol=1e-12)
    one = [np.array([17]), np.array([89])]
    out = decode_attention_sparse("fp4", enc, q, one, 0.2, H)
    for b, t in ((0, 17), (1, 89)):
        for h in range(H):
            v = F.fp4_decode(enc["v_codes"][b, h, t:t + 1], enc["v_scale"][b, h, t:t + 1])[0]
            np.testing.assert_allclose(out[b, h * G:(h + 1) * G], np.tile(v, (G, 1)), rtol=1e-12)
    sel = [np.array([0, 5, 6, 40, 88]), np.array([1, 2, 3, 60, 61])]
    compact = {k: np.stack([v[b][:, sel[b]] for b in range(B)]) for k, v in enc.items()}
    np.testing.assert_allclose(decode_attention_sparse("fp4", enc, q, sel, 0.2, H),
                               A.decode_attention("fp4", compact, q, [5, 5], 0.2, H), rtol=1e-12, atol=1e-12)
    assert not np.any(decode_attention_sparse("fp4", enc, q, [np.array([], int), sel[1]], 0.2, H)[0])


def test_sparse_decode_reads_kivi_staged_keys_like_dense():
    """Over every position, sparse decode with staged KIVI-2 keys is the staged
    dense decode; a selection of staged positions only uses the input keys."""
    rng = np.random.default_rng(8)
    B, H, T, d, G = 2, 2, 96, 64, 2
    K = rng.standard_normal((B, H, T, d))
    V = rng.standard_normal((B, H, T, d))
    enc = F.encode_cache("kivi2", K, V)
    q = rng.standard_normal((B, H * G, d))
    appended = np.array([80, 96])
    lens = appended
    full = [np.arange(80), np.arange(96)]
    got = decode_attention_sparse("kivi2", enc, q, full, 0.3, H, K_in=K, appended=appended)
    want = A.decode_attention_kivi_staged(enc, q[:, None], lens, 0.3, H, K, appended)[:, 0]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # positions 64..79 of sequence 0 are staged: their logits use K, not the codes
    sel = [np.array([64, 70, 79]), np.array([0, 95])]
    out = decode_attention_sparse("kivi2", enc, q, sel, 0.3, H, K_in=K, appended=appended)
    for h in range(H):
        qg = q[0, h * G:(h + 1) * G]
        lg = qg @ K[0, h, sel[0]].T * 0.3
        p = np.exp(lg - lg.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        vals = F.kivi2_decode_values(enc["v_codes"][0, h, sel[0]], enc["v_scale"][0, h, sel[0]],
                                     enc["v_zero"][0, h, sel[0]])
        np.testing.assert_allclose(out[0, h * G:(h + 1) * G], p @ vals, rtol=1e-12)
