"""Paged storage of a packed cache: where each token's bytes sit in a pool of
pages.  Test infrastructure, like the rest of oracle/: only the tests, the
smoke check and the benchmark's CPU baseline use it.

Reading (the pages say only that the kernels must work with paged attention --
page "TurboQuant vs OSCAR vs EpiCache", OSCAR's deployment list -- and that
paged allocators reclaim whole blocks -- page "How TriAttention cut LLM memory
use 10x", the paged-memory-fragmentation paragraph):
  * a page holds P consecutive positions of one sequence for every KV head;
  * a block table [B][J] names, for logical page j of sequence b (positions
    [j P, (j + 1) P)), the pool page p holding them;
  * pool element [p][h][s] of a per-token array is position j P + s of head h
    of that sequence (the latent has no head axis: [p][s]); per-group arrays
    (KIVI key scale and zero, one row per 32 tokens) hold P / 32 rows a page.
Nothing about the method's arithmetic changes: decode over a paged cache is
decode over the sequences these functions reassemble.
"""

import numpy as np


def sequences_from_pages(pool, table, heads=True):
    """Per-sequence arrays [B][H][J r][...] (heads=False: [B][J r][...]) from a
    pool [num_pages][H][r][...] ([num_pages][r][...]) with r rows a page."""
    pool = np.asarray(pool)
    table = np.asarray(table)
    axis = 1 if heads else 0
    return np.stack([np.concatenate([pool[p] for p in row], axis=axis) for row in table])


def pages_from_sequences(seqs, table, num_pages, heads=True):
    """The pool that holds per-sequence arrays under `table`; pages that no
    sequence names are zero."""
    seqs = np.asarray(seqs)
    table = np.asarray(table)
    J = table.shape[1]
    axis = 1 if heads else 0
    r = seqs.shape[axis + 1] // J
    shape = (num_pages,) + seqs.shape[1:axis + 1] + (r,) + seqs.shape[axis + 2:]
    pool = np.zeros(shape, dtype=seqs.dtype)
    for b in range(table.shape[0]):
        for j in range(J):
            part = seqs[b][:, j * r:(j + 1) * r] if heads else seqs[b][j * r:(j + 1) * r]
            pool[table[b, j]] = part
    return pool
