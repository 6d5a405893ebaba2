"""Hierarchical sparse indexing (HSI) and decode over the positions it selects.
Test infrastructure, like the rest of oracle/: only the tests, the smoke check
and the benchmark's CPU baseline use it.

Page "How DeepSeek-V4.1-Flash cut KV-cache storage by 4x via CSA2", HSI
section: the first (full-mode) layer scores every visible position, reduces the
scores to one maximum per block of 8 positions and keeps the best 2048 blocks,
a candidate pool of at most 16,384 positions; later (reindex-mode) layers score
only the pool's positions and keep the final top 512; attention then reads only
those.  The indexer that produces the scores is a trained model component and is
out of scope: scores are inputs.

Readings taken (the page gives the three steps and the sizes only):
  * scores are finite fp32 values compared as numbers (-0 equals +0); a block
    is positions [8 j, 8 j + 8) clipped to the sequence length L, its score the
    maximum over its positions below L;
  * "best" means largest; equal values rank the lower block index (lower pool
    entry) first, so the selection is unique;
  * the pool lists its positions in ascending order, the final selection too
    (its entries are positions, ascending);
  * when fewer blocks (pool entries) exist than asked for, all are kept;
  * decode over a selection is the plain decode attention restricted to the
    selected positions: softmax over their logits only.
"""

import numpy as np

from . import attention as A


def _rank_desc(values):
    """Indices ordered by value, largest first, equal values by lower index."""
    v = np.asarray(values, dtype=np.float32).astype(np.float64)  # fp32 values, exact in fp64
    return np.lexsort((np.arange(v.size), -v))


def block_maxima(scores, L, block=8):
    s = np.asarray(scores, dtype=np.float32)[:L]
    nb = -(-L // block)
    return np.array([s[j * block:min(L, (j + 1) * block)].max() for j in range(nb)], dtype=np.float32)


def candidate_pool(scores, L, block=8, top_blocks=2048):
    """int32 positions (ascending) of the top_blocks blocks with the largest maxima."""
    if L <= 0:
        return np.zeros(0, dtype=np.int32)
    m = block_maxima(scores, L, block)
    chosen = np.sort(_rank_desc(m)[:top_blocks])
    return np.array([t for j in chosen for t in range(j * block, min(L, (j + 1) * block))], dtype=np.int32)


def select_top_k(pool, pool_scores, k=512):
    """int32 positions (ascending) of the k pool entries with the largest scores."""
    pool = np.asarray(pool, dtype=np.int32)
    if pool.size == 0:
        return pool
    chosen = np.sort(_rank_desc(np.asarray(pool_scores)[:pool.size])[:k])
    return pool[chosen]


def decode_attention_sparse(fmt, cache, q, selections, scale, hkv, consts=None, latent_dim=512, K_in=None,
                            appended=None):
    """fp64 outputs [B, Hq, dv]: query (b, hq) attends over the positions
    selections[b] only (an empty selection gives zeros).  KIVI-2 with K_in
    ([B, H, T, d] input keys) and appended[b] tokens appended: keys of positions
    from the sequence's incomplete group on (32 * floor(appended[b] / 32)) are
    read from K_in, as dense decode reads its staged keys."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq = q.shape[:2]
    G = Hq // hkv
    dv = latent_dim if fmt == "latent" else q.shape[-1]
    out = np.zeros((B, Hq, dv))
    for b in range(B):
        sel = np.asarray(selections[b], dtype=np.int64)
        if sel.size == 0:
            continue
        for h in range(hkv):
            qg = q[b, h * G:(h + 1) * G]
            staged_from = 32 * (int(appended[b]) // 32) if K_in is not None else None

            def logit(t):
                if staged_from is not None and t >= staged_from:
                    return qg @ np.asarray(K_in[b, h, t:t + 1], np.float64).T
                return A._key_logits(fmt, cache, b, h, t, t + 1, qg, consts, latent_dim)
            logits = np.concatenate([logit(t) for t in sel], axis=1) * scale
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            vals = np.concatenate([A._values(fmt, cache, b, h, t, t + 1, consts, latent_dim) for t in sel], 0)
            o = p @ vals
            if fmt == "turbo":
                o = o @ np.asarray(consts["rot"], np.float64)
            out[b, h * G:(h + 1) * G] = o
    return out
