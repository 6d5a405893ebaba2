"""Pins for the paged-storage layout of the oracle: reassembly agrees with the
flat row formula of the layout (row ((p H + h) P + s) of a per-token array,
p = table[b][t // P], s = t mod P), round trips through a shuffled pool, and
leaves pages that no sequence names untouched."""

import numpy as np

from oracle.paging import pages_from_sequences, sequences_from_pages


def _table(rng, B, J, num_pages):
    return rng.permutation(num_pages)[:B * J].reshape(B, J).astype(np.int32)


def test_reassembly_matches_flat_row_formula():
    rng = np.random.default_rng(0)
    B, H, P, J, W, num_pages = 3, 2, 8, 4, 5, 15
    table = _table(rng, B, J, num_pages)
    pool = rng.integers(0, 256, size=(num_pages, H, P, W), dtype=np.uint8)
    seqs = sequences_from_pages(pool, table)
    flat = pool.reshape(-1, W)
    for b in range(B):
        for h in range(H):
            for t in range(J * P):
                row = (table[b, t // P] * H + h) * P + t % P
                np.testing.assert_array_equal(seqs[b, h, t], flat[row])
    # per-group rows: P / 32 rows a page, row ((p H + h) P / 32 + s / 32)
    Pg = 64
    gpool = rng.standard_normal((num_pages, H, Pg // 32, 3))
    gseq = sequences_from_pages(gpool, table)
    gflat = gpool.reshape(-1, 3)
    for t in range(0, J * Pg, 32):
        row = (table[1, t // Pg] * H + 1) * (Pg // 32) + (t % Pg) // 32
        np.testing.assert_array_equal(gseq[1, 1, t // 32], gflat[row])


def test_round_trip_and_unnamed_pages_zero():
    rng = np.random.default_rng(1)
    B, H, P, J, num_pages = 2, 3, 4, 3, 9
    table = _table(rng, B, J, num_pages)
    seqs = rng.standard_normal((B, H, J * P, 6))
    pool = pages_from_sequences(seqs, table, num_pages)
    assert pool.shape == (num_pages, H, P, 6)
    np.testing.assert_array_equal(sequences_from_pages(pool, table), seqs)
    unnamed = sorted(set(range(num_pages)) - set(table.ravel().tolist()))
    assert unnamed and not np.any(pool[unnamed])


def test_headless_layout():
    rng = np.random.default_rng(2)
    B, P, J, num_pages = 2, 4, 2, 5
    table = _table(rng, B, J, num_pages)
    seqs = rng.standard_normal((B, J * P, 7))
    pool = pages_from_sequences(seqs, table, num_pages, heads=False)
    assert pool.shape == (num_pages, P, 7)
    flat = pool.reshape(-1, 7)
    back = sequences_from_pages(pool, table, heads=False)
    np.testing.assert_array_equal(back, seqs)
    for t in range(J * P):
        np.testing.assert_array_equal(back[1, t], flat[table[1, t // P] * P + t % P])
