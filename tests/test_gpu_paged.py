"""GPU parity of paged storage: caches whose per-token buffers are a pool of
64-token pages named by a shuffled block table (with spare pages) must hold,
page by page, exactly the bytes a contiguous cache holds for the same appends,
and decode to the same outputs as the contiguous cache and within the 2e-3 row
bar of the oracle.  Covers every format, bulk, single-token and ragged appends,
KIVI key staging across pages, bf16 windows with a sink that is not a multiple
of 32 and several queries per sequence, and table entries outside the pool."""

import numpy as np
import pytest
import torch

import synth
from bit_kv_cache_04_amd import kvq
from bit_kv_cache_04_amd.kvq import BUFFERS
from gpu_helpers import (RTOL, host64, inputs, new_cache, oracle_constants, oracle_encode, row_rel_err,
                         softmax_scale)
from oracle import attention as OA
from oracle.paging import sequences_from_pages

pytestmark = pytest.mark.gpu

C = synth.CONFIGS
P = 64
SMALL = {
    "kivi2": C["kivi2_tiny"].scaled(batch=2, context=512),
    "fp4": C["fp4_b16_t32k"].scaled(batch=2, hq=8, hkv=2, context=1000),
    "turbo": C["turbo_b8_t128k"].scaled(batch=2, hq=16, hkv=2, context=777),
    "qjl1": C["qjl1_b1_t1m"].scaled(batch=2, hq=8, hkv=2, context=1500),
    "latent": C["latent_b64_t64k"].scaled(batch=2, hq=128, context=300),
}


def _table(B, per_seq, spare, seed):
    num_pages = B * per_seq + spare
    perm = np.random.default_rng(seed).permutation(num_pages)[:B * per_seq]
    return perm.reshape(B, per_seq).astype(np.int32), num_pages


def _pair(cfg, seed=0, **kw):
    """A paged cache (shuffled table, 5 spare pages) and a contiguous one."""
    cap = -(-cfg.context // P) * P
    table, num_pages = _table(cfg.batch, cap // P, 5, seed)
    paged = new_cache(cfg, capacity=cap, page_tokens=P, num_pages=num_pages, block_table=table, **kw)
    flat = new_cache(cfg, capacity=cap, **kw)
    return paged, flat, table


def _append(cache, cfg, K, V, t0, t1):
    if cfg.fmt == "latent":
        cache.append(K[:, t0:t1].contiguous(), None, t0)
    else:
        cache.append(K[:, :, t0:t1].contiguous(), V[:, :, t0:t1].contiguous(), t0)


def _assert_pages_equal(paged, flat, table, skip_pages=()):
    """Each sequence's pages, reassembled through the table, equal the contiguous
    cache's buffers (pages in skip_pages are not compared)."""
    heads = paged.fmt != "latent"
    for name in paged.bufs:
        if BUFFERS.index(name) >= BUFFERS.index("sink_k"):
            continue  # per-sequence windows and staging: not paged
        got = sequences_from_pages(paged.view(name).cpu().numpy(), table, heads=heads)
        want = flat.view(name).cpu().numpy()
        r = got.shape[2 if heads else 1] // table.shape[1]  # rows a page
        for b in range(table.shape[0]):
            for j in range(table.shape[1]):
                if (b, j) in skip_pages:
                    continue
                sl = (b, slice(None), slice(j * r, (j + 1) * r)) if heads else (b, slice(j * r, (j + 1) * r))
                bad = np.count_nonzero(got[sl].view(np.uint8) != want[sl].view(np.uint8))
                assert bad == 0, f"{paged.fmt} {name} sequence {b} page {j}: {bad} bytes differ"


@pytest.mark.parametrize("fmt", list(SMALL))
def test_paged_cache_matches_contiguous_and_oracle(fmt):
    cfg = SMALL[fmt]
    print(f"[paged] {fmt} {cfg}", flush=True)
    torch.manual_seed(0)
    paged, flat, table = _pair(cfg)
    K, V = inputs(cfg)
    T = cfg.context
    # a bulk append, an unaligned one (KIVI: keys staged across a page edge),
    # then single tokens up to the end
    cuts = [0, 256, T - 32 if fmt == "kivi2" else T - 3]
    for cache in (paged, flat):
        _append(cache, cfg, K, V, cuts[0], cuts[1])
        _append(cache, cfg, K, V, cuts[1], cuts[2] - (7 if fmt == "kivi2" else 0))
        for t in range(cuts[2] - (7 if fmt == "kivi2" else 0), T):
            _append(cache, cfg, K, V, t, t + 1)
    torch.cuda.synchronize()
    _assert_pages_equal(paged, flat, table)
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V) if V is not None else None, consts)
    q = synth.make_queries(cfg, device="cuda")
    lens = np.array([T, T // 2 + 7], dtype=np.int32)
    if fmt == "kivi2":
        lens[1] = 288  # whole coded groups for the plain oracle
    lt = torch.from_numpy(lens).cuda()
    out_p = paged.decode(q, lt, softmax_scale(cfg)).cpu().numpy()
    # KIVI-2's matrix-core kernel reads contiguous caches only, so a paged KIVI-2
    # cache takes the fp32 kernel: the contiguous cache is compared on that
    # kernel too, and its own matrix-core output against the oracle below
    flags = kvq.DECODE_FP32 if fmt == "kivi2" else 0
    out_f = flat.decode(q, lt, softmax_scale(cfg), flags=flags).cpu().numpy()
    np.testing.assert_array_equal(out_p, out_f)
    ref = OA.decode_attention(fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, consts,
                              latent_dim=cfg.head_dim)
    err = row_rel_err(out_p, ref)
    if fmt == "kivi2":
        out_m = flat.decode(q, lt, softmax_scale(cfg)).cpu().numpy()
        err = np.maximum(err, row_rel_err(out_m, ref))
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


@pytest.mark.parametrize("fmt,nq", [("fp4", 3), ("qjl1", 1), ("kivi2", 2), ("turbo", 1), ("turbo", 2)])
def test_paged_windows_and_queries(fmt, nq):
    """bf16 sink (40 tokens: matrix-core tiles start at 32 and mask 32..39) and
    recent windows over a paged history, sequences appended to ragged lengths
    through one-sequence views, last tokens one at a time."""
    cfg = SMALL[fmt]
    sink, recent = 40, 100
    print(f"[paged windows] {fmt} nq={nq}", flush=True)
    torch.manual_seed(0)
    paged, flat, table = _pair(cfg, seed=1, sink_tokens=sink, recent_tokens=recent)
    K, V = inputs(cfg)
    lens = np.array([cfg.context, cfg.context // 2 + 13], dtype=np.int32)
    for cache in (paged, flat):
        for b in range(cfg.batch):
            seq, L = cache.sequence(b), int(lens[b])
            seq.append(K[b:b + 1, :, :L - 4].contiguous(), V[b:b + 1, :, :L - 4].contiguous(), 0)
            for t in range(L - 4, L):
                seq.append(K[b:b + 1, :, t:t + 1].contiguous(), V[b:b + 1, :, t:t + 1].contiguous(), t)
    torch.cuda.synchronize()
    _assert_pages_equal(paged, flat, table)
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V), consts)
    q = synth.make_queries(cfg.scaled(hq=nq * cfg.hq), device="cuda").view(cfg.batch, nq, cfg.hq, -1)
    lt = torch.from_numpy(lens).cuda()
    out_p = paged.decode(q, lt, softmax_scale(cfg)).cpu().numpy()
    out_f = flat.decode(q, lt, softmax_scale(cfg)).cpu().numpy()
    np.testing.assert_array_equal(out_p, out_f)
    ref = OA.decode_attention_mixed(fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, host64(K), host64(V),
                                    sink, recent, consts)
    err = row_rel_err(out_p.reshape(-1, out_p.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


@pytest.mark.parametrize("fmt", ["fp4", "kivi2", "turbo", "latent"])
def test_paged_ragged_appends(fmt):
    """One append with a first position per sequence lands in each sequence's
    own pages."""
    cfg = SMALL[fmt].scaled(context=320)
    print(f"[paged ragged] {fmt}", flush=True)
    paged, flat, table = _pair(cfg, seed=2)
    K, V = inputs(cfg)
    n = 64
    starts = [0, 96]
    for cache in (paged, flat):
        if fmt == "latent":
            cache.append(K[:, :n].contiguous(), None, starts)
            cache.append(K[:, n:2 * n].contiguous(), None, [s + n for s in starts])
        else:
            cache.append(K[:, :, :n].contiguous(), V[:, :, :n].contiguous(), starts)
            cache.append(K[:, :, n:2 * n].contiguous(), V[:, :, n:2 * n].contiguous(), [s + n for s in starts])
    torch.cuda.synchronize()
    _assert_pages_equal(paged, flat, table)


@pytest.mark.parametrize("fmt", ["fp4", "turbo"])
def test_table_entries_outside_the_pool(fmt):
    """An entry outside [0, num_pages) is never followed: appends to it are
    dropped, every other page is written as usual, and decode of a prefix that
    stays clear of it is unchanged."""
    cfg = SMALL[fmt].scaled(context=512)
    print(f"[paged out-of-pool] {fmt}", flush=True)
    paged, flat, table = _pair(cfg, seed=3)
    bad = table.copy()
    bad[1, -1] = paged.num_pages + 7
    bad[0, 2] = -1
    paged.table.copy_(torch.from_numpy(bad))
    K, V = inputs(cfg)
    for cache in (paged, flat):
        _append(cache, cfg, K, V, 0, cfg.context)
    torch.cuda.synchronize()
    gather = np.where((bad >= 0) & (bad < paged.num_pages), bad, 0)  # bad entries read page 0, not compared
    _assert_pages_equal(paged, flat, gather, skip_pages={(1, bad.shape[1] - 1), (0, 2)})
    # the pages the bad entries would have named in the original table stay zero
    for name in paged.bufs:
        pool = paged.view(name).cpu().numpy()
        for p in (table[1, -1], table[0, 2]):
            assert not np.any(pool[p].view(np.uint8)), (name, p)
    q = synth.make_queries(cfg, device="cuda")
    lens = np.array([2 * P, cfg.context - P], dtype=np.int32)  # clear of both bad pages
    lt = torch.from_numpy(lens).cuda()
    out_p = paged.decode(q, lt, softmax_scale(cfg)).cpu().numpy()
    out_f = flat.decode(q, lt, softmax_scale(cfg)).cpu().numpy()
    np.testing.assert_array_equal(out_p, out_f)
    # a decode that meets a bad page completes (its output is unspecified)
    full = torch.full((cfg.batch,), cfg.context, dtype=torch.int32, device="cuda")
    paged.decode(q, full, softmax_scale(cfg))
    torch.cuda.synchronize()


@pytest.mark.parametrize("page,cap", [(32, 64), (64, 64)])
def test_paged_ragged_beyond_one_launch(page, cap):
    """300 sequences (two launches of at most 256, the block table shifted for the
    second), ragged starts, the smallest page and one page per sequence."""
    cfg = C["fp4_b16_t32k"].scaled(batch=300, hq=1, hkv=1, context=cap)
    print(f"[paged 300] page={page} cap={cap}", flush=True)
    per_seq = cap // page
    table, num_pages = _table(300, per_seq, 7, seed=page)
    paged = new_cache(cfg, capacity=cap, page_tokens=page, num_pages=num_pages, block_table=table)
    flat = new_cache(cfg, capacity=cap)
    K, V = synth.make_kv(cfg, 0, 300, 0, 3, device="cuda")
    starts = np.random.default_rng(5).integers(0, cap - 3, 300).tolist()
    for cache in (paged, flat):
        cache.append(K.contiguous(), V.contiguous(), starts)
    torch.cuda.synchronize()
    _assert_pages_equal(paged, flat, table)
    q = synth.make_queries(cfg, device="cuda")
    lens = torch.from_numpy(np.array(starts, np.int32) + 3).cuda()
    np.testing.assert_array_equal(paged.decode(q, lens, softmax_scale(cfg)).cpu().numpy(),
                                  flat.decode(q, lens, softmax_scale(cfg)).cpu().numpy())


@pytest.mark.parametrize("fmt,nq", [("turbo", 2), ("latent", 3), ("qjl1", 4)])
def test_paged_multi_query(fmt, nq):
    """Several queries per sequence on paged caches: the per-query launches of the
    TurboQuant and latent kernels, and the QJL columns, read through the table."""
    cfg = SMALL[fmt]
    print(f"[paged multi-query] {fmt} nq={nq}", flush=True)
    paged, flat, table = _pair(cfg, seed=6)
    K, V = inputs(cfg)
    for cache in (paged, flat):
        _append(cache, cfg, K, V, 0, cfg.context)
    torch.cuda.synchronize()
    q = synth.make_queries(cfg.scaled(hq=nq * cfg.hq), device="cuda").view(cfg.batch, nq, cfg.hq, -1)
    lens = np.array([cfg.context, cfg.context // 3], dtype=np.int32)
    lt = torch.from_numpy(lens).cuda()
    out_p = paged.decode(q, lt, softmax_scale(cfg)).cpu().numpy()
    out_f = flat.decode(q, lt, softmax_scale(cfg)).cpu().numpy()
    np.testing.assert_array_equal(out_p, out_f)
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V) if V is not None else None, consts)
    ref = OA.decode_attention_multi(fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, consts,
                                    latent_dim=cfg.head_dim)
    err = row_rel_err(out_p.reshape(-1, out_p.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL
