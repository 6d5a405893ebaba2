"""GPU parity of hierarchical sparse indexing and sparse decode through the C
ABI: the candidate pool and the reindex top-k must equal the oracle's positions
exactly (ties included), and decode over selected positions must stay within
the 2e-3 row bar of the oracle for every format."""

import numpy as np
import pytest
import torch

import synth
from bit_kv_cache_04_amd.cache import hsi_candidates, hsi_select
from gpu_helpers import RTOL, host64, inputs, new_cache, oracle_constants, oracle_encode, row_rel_err, softmax_scale
from oracle.hsi import candidate_pool, decode_attention_sparse, select_top_k

pytestmark = pytest.mark.gpu


def _ties(x, step):
    return torch.round(x / step) * step  # coarse scores: many equal values


@pytest.mark.parametrize("S,lens,block,top,step", [
    (5000, [5000, 1234, 7, 0], 8, 100, 0.25),
    (5000, [4999, 5000, 17, 8], 8, 2048, 0.0),
    (3000, [3000, 2999, 1], 4, 1, 0.5),
    (70000, [70000, 65536, 123], 8, 2048, 0.125),
    (1 << 20, [1 << 20], 8, 2048, 0.0),
    (1 << 17, [131071], 16, 5000, 0.0),
    (200000, [200000, 150001, 17, 0], 8, 2048, 0.25),   # > 16,384 blocks: many workgroups per sequence
    (300000, [299999, 70000], 8, 40000, 0.0),           # every block of the shorter sequence kept
])
def test_candidate_pool_matches_oracle(S, lens, block, top, step):
    B = len(lens)
    print(f"[hsi pool] S={S} lens={lens} block={block} top={top} step={step}", flush=True)
    scores = synth.make_indexer_scores(7, B, S, device="cuda")
    if step:
        scores = _ties(scores, step)
    scores[0, 0] = -0.0
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    pool, pool_n = hsi_candidates(scores, lt, block, top)
    pool, pool_n = pool.cpu().numpy(), pool_n.cpu().numpy()
    host = scores.cpu().numpy()
    for b in range(B):
        want = candidate_pool(host[b], lens[b], block, top)
        assert pool_n[b] == want.size, (b, pool_n[b], want.size)
        np.testing.assert_array_equal(pool[b, :want.size], want)


@pytest.mark.parametrize("S,top_blocks,k,step", [(70000, 2048, 512, 0.0), (70000, 2048, 512, 0.25),
                                                 (9000, 300, 512, 0.0), (70000, 4096, 512, 0.5),
                                                 (5000, 64, 1, 0.0), (300000, 4096, 3000, 0.0)])
def test_reindex_top_k_matches_oracle(S, top_blocks, k, step):
    """Pools up to 16,384 entries are staged in LDS, larger ones read in place."""
    B = 3
    print(f"[hsi select] S={S} top_blocks={top_blocks} k={k} step={step}", flush=True)
    lens = [S, S // 2 + 3, 1000]
    scores = synth.make_indexer_scores(11, B, S, device="cuda")
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    pool, pool_n = hsi_candidates(scores, lt, 8, top_blocks)
    ps = synth.make_indexer_scores(12, B, top_blocks * 8, layer=1, device="cuda")
    if step:
        ps = _ties(ps, step)
    sel, sel_n = hsi_select(ps, pool, pool_n, k)
    pool_h, pn, ps_h = pool.cpu().numpy(), pool_n.cpu().numpy(), ps.cpu().numpy()
    sel_h, sn = sel.cpu().numpy(), sel_n.cpu().numpy()
    for b in range(B):
        want = select_top_k(pool_h[b, :pn[b]], ps_h[b, :pn[b]], k)
        assert sn[b] == want.size
        np.testing.assert_array_equal(sel_h[b, :want.size], want)


SMALL = {
    "kivi2": synth.CONFIGS["kivi2_tiny"].scaled(batch=2, context=512),
    "fp4": synth.CONFIGS["fp4_b16_t32k"].scaled(batch=2, hq=8, hkv=2, context=1000),
    "turbo": synth.CONFIGS["turbo_b8_t128k"].scaled(batch=2, hq=16, hkv=2, context=777),
    "qjl1": synth.CONFIGS["qjl1_b1_t1m"].scaled(batch=2, hq=8, hkv=2, context=1500),
    "latent": synth.CONFIGS["latent_b64_t64k"].scaled(batch=2, hq=128, context=3000),
}


@pytest.mark.parametrize("fmt", list(SMALL))
def test_sparse_decode_matches_oracle(fmt):
    """Selections of different sizes per sequence (one empty), with entries
    outside the cache that must be skipped, across several tiles and splits."""
    cfg = SMALL[fmt]
    print(f"[sparse decode] {fmt}", flush=True)
    torch.manual_seed(0)
    cache = new_cache(cfg)
    K, V = inputs(cfg)
    if fmt == "latent":
        cache.append(K, None, 0)
    else:
        cache.append(K, V, 0)
    T = cfg.context
    rng = np.random.default_rng(3)
    K_cap = 300
    sel = np.full((cfg.batch, K_cap), -1, np.int32)
    picks = [np.sort(rng.choice(T, 200, replace=False)), np.sort(rng.choice(T, 37, replace=False))]
    sel[0, :200] = picks[0]
    sel[1, :37] = picks[1]
    sel[1, 37:40] = [T + 5, -3, cfg.context * 4]       # skipped
    n = np.array([200, 40], np.int32)
    q = synth.make_queries(cfg, device="cuda")
    out = cache.decode_sparse(q, torch.from_numpy(sel).cuda(), torch.from_numpy(n).cuda(), softmax_scale(cfg))
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V) if V is not None else None, consts)
    ref = decode_attention_sparse(fmt, enc, host64(q), picks, softmax_scale(cfg), cfg.hkv, consts,
                                  latent_dim=cfg.head_dim)
    err = row_rel_err(out.cpu().numpy(), ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL
    # an empty selection gives zeros
    z = cache.decode_sparse(q, torch.from_numpy(sel).cuda(), torch.zeros(cfg.batch, dtype=torch.int32,
                                                                          device="cuda"), softmax_scale(cfg))
    assert not torch.any(z)


def test_hsi_pipeline_on_latent_cache():
    """Full mode, reindex mode and sparse decode chained on a latent cache."""
    cfg = synth.CONFIGS["latent_b64_t64k"].scaled(batch=2, hq=64, context=20000)
    print("[hsi pipeline] latent", flush=True)
    cache = new_cache(cfg)
    K, _ = inputs(cfg)
    cache.append(K, None, 0)
    lens = [20000, 9001]
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    full = synth.make_indexer_scores(21, cfg.batch, cfg.context, device="cuda")
    pool, pool_n = hsi_candidates(full, lt, 8, 2048)
    ps = synth.make_indexer_scores(22, cfg.batch, 2048 * 8, layer=1, device="cuda")
    sel, sel_n = hsi_select(ps, pool, pool_n, 512)
    q = synth.make_queries(cfg, device="cuda")
    out = cache.decode_sparse(q, sel, sel_n, softmax_scale(cfg)).cpu().numpy()
    fh, psh = full.cpu().numpy(), ps.cpu().numpy()
    picks = []
    for b in range(cfg.batch):
        p = candidate_pool(fh[b], lens[b], 8, 2048)
        picks.append(select_top_k(p, psh[b, :p.size], 512))
        np.testing.assert_array_equal(sel.cpu().numpy()[b, :picks[b].size], picks[b])
    enc = oracle_encode(cfg, host64(K), None, {})
    ref = decode_attention_sparse("latent", enc, host64(q), picks, softmax_scale(cfg), cfg.hkv, {},
                                  latent_dim=cfg.head_dim)
    err = row_rel_err(out, ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


@pytest.mark.parametrize("hq,n,cap", [(32, 1500, 1600), (128, 40, 64), (64, 700, 700), (128, 512, 512)])
def test_sparse_latent_kernel_shapes(hq, n, cap):
    """The latent matrix-core kernel's gather mode: 1, 2 and 4 waves, selections
    longer than one split's 512 staged positions, ragged tiles and invalid slots."""
    cfg = synth.CONFIGS["latent_b64_t64k"].scaled(batch=2, hq=hq, context=4000)
    print(f"[sparse latent] hq={hq} n={n} cap={cap}", flush=True)
    cache = new_cache(cfg)
    K, _ = inputs(cfg)
    cache.append(K, None, 0)
    rng = np.random.default_rng(hq + n)
    sel = np.full((cfg.batch, cap), -1, np.int32)
    picks = []
    for b, m in enumerate((n, max(1, n // 3))):
        p = np.sort(rng.choice(cfg.context, m, replace=False)).astype(np.int32)
        sel[b, :m] = p
        if m < cap:
            sel[b, m] = cfg.context + 77  # outside the cache: skipped
        picks.append(p)
    lens = np.array([n, min(cap, max(1, n // 3) + 1)], np.int32)
    q = synth.make_queries(cfg, device="cuda")
    out = cache.decode_sparse(q, torch.from_numpy(sel).cuda(), torch.from_numpy(lens).cuda(), softmax_scale(cfg))
    enc = oracle_encode(cfg, host64(K), None, {})
    ref = decode_attention_sparse("latent", enc, host64(q), picks, softmax_scale(cfg), cfg.hkv, {},
                                  latent_dim=cfg.head_dim)
    err = row_rel_err(out.cpu().numpy(), ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


@pytest.mark.parametrize("fmt,G,n", [("fp4", 1, 1500), ("fp4", 16, 700), ("qjl1", 8, 600), ("fp4", 2, 40),
                                     ("qjl1", 1, 513), ("turbo", 8, 1500), ("turbo", 1, 300), ("turbo", 4, 64)])
def test_sparse_mfma_kernel_shapes(fmt, G, n):
    """The FP4 / QJL and TurboQuant matrix-core kernels' gather modes: query-group sizes, several
    splits of up to 512 staged positions, ragged tiles and skipped entries."""
    cfg = SMALL[fmt].scaled(hq=2 * G, hkv=2, context=3000)
    print(f"[sparse mfma] {fmt} G={G} n={n}", flush=True)
    cache = new_cache(cfg)
    K, V = inputs(cfg)
    cache.append(K, V, 0)
    rng = np.random.default_rng(G * 1000 + n)
    cap = n + 8
    sel = np.full((cfg.batch, cap), -1, np.int32)
    picks = [np.sort(rng.choice(cfg.context, n, replace=False)).astype(np.int32),
             np.sort(rng.choice(cfg.context, max(1, n // 5), replace=False)).astype(np.int32)]
    for b, p in enumerate(picks):
        sel[b, :p.size] = p
    sel[1, picks[1].size] = cfg.context + 3  # outside the cache: skipped
    lens = np.array([n, picks[1].size + 1], np.int32)
    q = synth.make_queries(cfg, device="cuda")
    out = cache.decode_sparse(q, torch.from_numpy(sel).cuda(), torch.from_numpy(lens).cuda(), softmax_scale(cfg))
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V), consts)
    ref = decode_attention_sparse(fmt, enc, host64(q), picks, softmax_scale(cfg), cfg.hkv, consts)
    err = row_rel_err(out.cpu().numpy(), ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


@pytest.mark.parametrize("fmt", ["fp4", "latent"])
def test_sparse_decode_on_paged_cache(fmt):
    """A paged cache (shuffled 64-token pages) takes sparse decode on the general
    kernel, which looks each slot's row up through the block table."""
    cfg = SMALL[fmt].scaled(context=1024)
    print(f"[sparse paged] {fmt}", flush=True)
    per_seq = cfg.context // 64
    table = np.random.default_rng(9).permutation(cfg.batch * per_seq + 3)[:cfg.batch * per_seq]
    cache = new_cache(cfg, page_tokens=64, num_pages=cfg.batch * per_seq + 3,
                      block_table=table.reshape(cfg.batch, per_seq))
    K, V = inputs(cfg)
    if fmt == "latent":
        cache.append(K, None, 0)
    else:
        cache.append(K, V, 0)
    rng = np.random.default_rng(4)
    picks = [np.sort(rng.choice(cfg.context, 300, replace=False)).astype(np.int32),
             np.sort(rng.choice(cfg.context, 77, replace=False)).astype(np.int32)]
    sel = np.full((cfg.batch, 300), -1, np.int32)
    for b, p in enumerate(picks):
        sel[b, :p.size] = p
    n = np.array([p.size for p in picks], np.int32)
    q = synth.make_queries(cfg, device="cuda")
    out = cache.decode_sparse(q, torch.from_numpy(sel).cuda(), torch.from_numpy(n).cuda(), softmax_scale(cfg))
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V) if V is not None else None, consts)
    ref = decode_attention_sparse(fmt, enc, host64(q), picks, softmax_scale(cfg), cfg.hkv, consts,
                                  latent_dim=cfg.head_dim)
    err = row_rel_err(out.cpu().numpy(), ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


def test_hsi_degenerate_cases():
    """Block sizes 1 and 64, every score equal (the lowest blocks win), lengths
    past the score row (clipped) or negative (empty), an empty pool, and a
    selection asked for more entries than the pool holds."""
    S, B = 3000, 4
    lens = [S + 500, -7, 64, 2999]
    eff = [min(max(x, 0), S) for x in lens]
    flat = torch.full((B, S), 1.5, dtype=torch.float32, device="cuda")
    rnd = synth.make_indexer_scores(5, B, S, device="cuda")
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for scores in (flat, rnd):
        host = scores.cpu().numpy()
        for block, top in ((1, 700), (64, 5), (64, 1), (8, 1)):
            print(f"[hsi degenerate] block={block} top={top}", flush=True)
            pool, pool_n = hsi_candidates(scores, lt, block, top)
            pool_h, pn = pool.cpu().numpy(), pool_n.cpu().numpy()
            for b in range(B):
                want = candidate_pool(host[b], eff[b], block, top)
                assert pn[b] == want.size
                np.testing.assert_array_equal(pool_h[b, :want.size], want)
            ps = torch.full((B, top * block), -2.0, dtype=torch.float32, device="cuda")
            sel, sel_n = hsi_select(ps, pool, pool_n, 1000)
            sel_h, sn = sel.cpu().numpy(), sel_n.cpu().numpy()
            for b in range(B):
                want = select_top_k(pool_h[b, :pn[b]], ps.cpu().numpy()[b, :pn[b]], 1000)
                assert sn[b] == want.size
                np.testing.assert_array_equal(sel_h[b, :want.size], want)


def test_sparse_decode_kivi_staged_positions():
    """KIVI-2 sequences with an incomplete last key group: selected positions in
    it are read from the staged keys, the others from the codes."""
    cfg = SMALL["kivi2"].scaled(batch=2, context=512)
    print("[sparse kivi staged]", flush=True)
    cache = new_cache(cfg)
    K, V = inputs(cfg)
    appended = [500, 451]
    for b, A_ in enumerate(appended):
        seq = cache.sequence(b)
        seq.append(K[b:b + 1, :, :448].contiguous(), V[b:b + 1, :, :448].contiguous(), 0)
        seq.append(K[b:b + 1, :, 448:A_].contiguous(), V[b:b + 1, :, 448:A_].contiguous(), 448)
    torch.cuda.synchronize()
    picks = [np.array([3, 100, 447, 470, 479, 480, 481, 499], np.int32),
             np.array([0, 447, 448, 449, 450], np.int32)]
    sel = np.full((cfg.batch, 8), -1, np.int32)
    for b, p in enumerate(picks):
        sel[b, :p.size] = p
    n = np.array([p.size for p in picks], np.int32)
    q = synth.make_queries(cfg, device="cuda")
    out = cache.decode_sparse(q, torch.from_numpy(sel).cuda(), torch.from_numpy(n).cuda(), softmax_scale(cfg))
    enc = oracle_encode(cfg, host64(K), host64(V), {})
    ref = decode_attention_sparse("kivi2", enc, host64(q), picks, softmax_scale(cfg), cfg.hkv, {},
                                  K_in=host64(K), appended=appended)
    err = row_rel_err(out.cpu().numpy(), ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL
