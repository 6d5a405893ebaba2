"""Decode-attention bandwidth benchmark for the packed low-bit KV cache.

One step = the whole hot path for one decode token of every sequence: append
that token's K/V into the packed cache (the format's pack kernel) and run
single-query attention over the full context (query prep, split-context
attention, merge), at a fixed context length.

The timed region replays the step as a HIP graph (captured once after the
warm-up and checked bit for bit against the eager step); the attention kernel's
own duration, for the roofline, comes from HIP events around its launches in
an eager pass over the same number of steps.

Prints one JSON line.  `value` is decode KV GB/s: the packed bytes the
attention reads per step (codes + scales/norms of every cached token) over the
measured step time.  The default workload is FP4 E2M1 with one bf16 scale per
16 channels, batch 16, 32 query / 8 KV heads, head dim 128, 32768 tokens.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_VALU_PEAK_TFLOPS = 157.3  # fp32 vector peak (256 CUs, 2.4 GHz)
HBM_PEAK_GBS = 8000.0


def counted_bytes(cfg, lib_layout, kvq, sink=0, recent=0):
    """Packed KV + scales/norms read by one decode step over cfg.context tokens
    (with bf16 sink / recent windows: those tokens as bf16 K and V instead)."""
    per_tok = kvq.kv_bytes_per_token(lib_layout, 1)
    window = min(cfg.context, sink + recent)
    return (per_tok * cfg.batch * (cfg.context - window)
            + cfg.batch * cfg.hkv * window * cfg.head_dim * 2 * 2)


def cpu_baseline(cfg, budget_s=12.0, rotation="haar", hsi=False):
    """Time the oracle's decode on a bounded sample: one (sequence, KV head) unit at a time
    (hsi: the oracle's candidate pool, reindex top-k and decode over the selection)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import attention as OA
    from oracle import formats as OF
    from oracle.bytes import per_token_head
    from oracle.lloyd_max import canonical_codebook
    from oracle.rotation import canonical_hadamard_rotation, canonical_projection, canonical_rotation

    T = cfg.context
    unit = cfg.scaled(batch=1, hkv=1, hq=cfg.group)
    consts = {}
    if cfg.fmt == "turbo":
        if rotation == "haar":
            consts["rot"] = canonical_rotation(synth.gaussian_matrix(cfg.seed, cfg.head_dim, cfg.head_dim, stream=1))
        else:
            consts["rot"] = canonical_hadamard_rotation(cfg.head_dim, rotation == "hadamard")
        consts["levels"], consts["thresholds"] = canonical_codebook(2, cfg.head_dim)
    if cfg.fmt in ("turbo", "qjl1"):
        consts["proj"] = canonical_projection(synth.gaussian_matrix(cfg.seed, 128, cfg.head_dim, stream=2))
    enc_parts = []
    for t0 in range(0, T, 65536):
        t1 = min(T, t0 + 65536)
        if cfg.fmt == "latent":
            lat = synth.make_latent(unit, 0, 1, t0, t1, device="cpu").float().numpy().astype(np.float64)
            enc_parts.append(OF.encode_cache("latent", latent=lat, latent_dim=cfg.head_dim))
        else:
            K, V = synth.make_kv(unit, 0, 1, t0, t1, device="cpu")
            enc_parts.append(OF.encode_cache(cfg.fmt, K.float().numpy().astype(np.float64),
                                             V.float().numpy().astype(np.float64), consts=consts))
    axis = 1 if cfg.fmt == "latent" else 2
    enc = {k: np.concatenate([e[k] for e in enc_parts], axis=axis) for k in enc_parts[0]}
    q = synth.make_queries(unit, device="cpu").float().numpy().astype(np.float64)
    scale = 1.0 / math.sqrt(cfg.key_width)
    units = 0
    if hsi:
        from oracle.hsi import candidate_pool, decode_attention_sparse, select_top_k
        full = synth.make_indexer_scores(cfg.seed, 1, T).numpy()[0]
        pool_scores = synth.make_indexer_scores(cfg.seed, 1, 8 * 2048, layer=1).numpy()[0]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            if hsi:
                pool = candidate_pool(full, T, 8, 2048)
                sel = select_top_k(pool, pool_scores[:pool.size], 512)
                decode_attention_sparse(cfg.fmt, enc, q, [sel], scale, 1, consts, latent_dim=cfg.head_dim)
            else:
                OA.decode_attention(cfg.fmt, enc, q, [T], scale, 1, consts, latent_dim=cfg.head_dim)
            units += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    if hsi:
        nbytes = units * (4 * (T + 8 * 2048) + 512 * per_token_head(cfg.fmt, cfg.head_dim, cfg.rope_dim))
        return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{units} x HSI pool + top-512 + sparse decode of 1 sequence x 1 KV head "
                          f"({unit.hq} q heads) over {T} tokens, fp64 numpy on 1 thread, {el:.1f} s"}
    nbytes = units * T * per_token_head(cfg.fmt, cfg.head_dim, cfg.rope_dim)
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{units} x decode of 1 sequence x 1 KV head ({unit.hq} q heads) over {T} tokens, "
                      f"fp64 numpy on 1 thread, {el:.1f} s"}


MFMA_F16_PEAK_TFLOPS = 2500.0


def measured_traffic(workload):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary (profiles/*_<workload>_pmc.txt: FETCH_SIZE and WRITE_SIZE scaled by a
    plain copy of known size), or None when there is none or the kernel's source
    has changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_pmc.txt"))):
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        src = os.path.join(ROOT, kv.get("source", ""))
        if not os.path.isfile(src) or "traffic_bytes_per_launch" not in kv:
            continue
        if hashlib.sha256(open(src, "rb").read()).hexdigest() == kv.get("source_sha256"):
            return int(kv["traffic_bytes_per_launch"])
    return None


def roofline(cfg, nbytes, dec_ms, nq=1, windowed=False, paged=False):
    """Roofline of the split-context attention kernel, timed by events around its launch.
    The counter summaries cover the one-query kernels: traffic is None for nq > 1."""
    traffic = measured_traffic(cfg.name) if nq == 1 and not windowed and not paged else None
    if cfg.fmt == "latent":
        # 128 heads x (576 + 512) x 2 flop per token: a dense contraction on fp16 matrix cores
        flops = 2.0 * nq * cfg.batch * cfg.context * cfg.hq * (cfg.key_width + cfg.head_dim)
        ach = flops / (dec_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": "split-context attention", "kernel_us": round(dec_ms * 1e3, 2),
                "hbm_gbs": round(nbytes / (dec_ms * 1e-3) / 1e9, 2)}
    ach = nbytes / (dec_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "split-context attention", "kernel_us": round(dec_ms * 1e3, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="fp4_b16_t32k")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--sink", type=int, default=0, help="leading tokens kept bf16 (FP4-valued formats)")
    ap.add_argument("--recent", type=int, default=0, help="trailing tokens kept bf16 (FP4-valued formats)")
    ap.add_argument("--queries", type=int, default=1,
                    help="query tokens per sequence (drafted positions checked in one pass); the step "
                         "appends that many tokens")
    ap.add_argument("--rotation", default="haar", choices=["haar", "hadamard", "hadamard_plain"],
                    help="TurboQuant rotation: a Haar draw, or the Hadamard transform with (or without) "
                         "the bit-reversal permutation")
    ap.add_argument("--page-tokens", type=int, default=0,
                    help="paged storage: tokens per page, the pool's pages assigned to sequences in a seeded "
                         "shuffled order")
    ap.add_argument("--hsi", action="store_true",
                    help="hierarchical sparse indexing: candidate pool (top 2048 blocks of 8 by synthetic full-mode "
                         "scores), reindex top 512 (synthetic pool scores), decode over the selected positions")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph replay")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode shards by sequence and KV head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from bit_kv_cache_04_amd import kvq
    from bit_kv_cache_04_amd.cache import PackedKVCache, make_constants

    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    consts = None
    if cfg.fmt in ("turbo", "qjl1"):
        consts = make_constants(cfg.fmt, cfg.head_dim,
                                synth.gaussian_matrix(cfg.seed, cfg.head_dim, cfg.head_dim, stream=1),
                                synth.gaussian_matrix(cfg.seed, 128, cfg.head_dim, stream=2),
                                rotation=args.rotation if cfg.fmt == "turbo" else "haar")
    paging = {}
    if args.page_tokens:
        import numpy as np
        per_seq = cfg.context // args.page_tokens
        table = np.random.default_rng(cfg.seed).permutation(cfg.batch * per_seq).reshape(cfg.batch, per_seq)
        paging = dict(page_tokens=args.page_tokens, num_pages=cfg.batch * per_seq, block_table=table)
    cache = PackedKVCache(cfg.fmt, cfg.batch, cfg.hkv, cfg.head_dim, cfg.context, cfg.rope_dim, device=dev,
                          constants=consts, sink_tokens=args.sink, recent_tokens=args.recent, **paging)
    T = cfg.context
    # prefill the first T - n tokens (untimed), one sequence and 16K tokens at a
    # time to bound input memory
    # KIVI keys are quantised per whole 32-token group, so its step appends one group
    nq = args.queries
    n_new = 32 if cfg.fmt == "kivi2" else max(nq, cfg.append_new)
    n_pre = T - n_new
    for b in range(cfg.batch):
        seq = cache.sequence(b)
        for t0 in range(0, n_pre, 16384):
            t1 = min(n_pre, t0 + 16384)
            if cfg.fmt == "latent":
                seq.append(synth.make_latent(cfg, b, b + 1, t0, t1, device=dev), None, t0)
            else:
                K, V = synth.make_kv(cfg, b, b + 1, t0, t1, device=dev)
                seq.append(K, V, t0)
    # the tokens appended inside every step: the decode token at T-1, or for a
    # bulk-append workload the last `append_new` tokens of the context
    if cfg.fmt == "latent":
        k_new, v_new = synth.make_latent(cfg, 0, cfg.batch, T - n_new, T, device=dev), None
    else:
        k_new, v_new = synth.make_kv(cfg, 0, cfg.batch, T - n_new, T, device=dev)
    q = synth.make_queries(cfg, device=dev)
    if nq > 1:
        q = synth.make_queries(cfg.scaled(hq=nq * cfg.hq), device=dev).view(cfg.batch, nq, cfg.hq, -1)
    lens = torch.full((cfg.batch,), T, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(cfg.key_width)
    out = torch.empty(*q.shape[:-1], cfg.head_dim, dtype=torch.float32, device=dev)
    ws = torch.zeros(cache.workspace_bytes(cfg.hq, T, args.splits, q.dtype, nq), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:  # torch creates the HIP event on first record; the library records it afterwards
        a.record()
        b.record()

    if args.hsi:
        from bit_kv_cache_04_amd.cache import hsi_candidates, hsi_select
        if nq != 1 or args.sink or args.recent:
            raise SystemExit("bench.py: --hsi takes one query per sequence and no bf16 windows")
        HSI_BLOCK, HSI_TOP_BLOCKS, HSI_TOP_K = 8, 2048, 512
        pool_cap = HSI_BLOCK * HSI_TOP_BLOCKS
        full_scores = synth.make_indexer_scores(cfg.seed, cfg.batch, T, device=dev)
        pool_scores = synth.make_indexer_scores(cfg.seed, cfg.batch, pool_cap, layer=1, device=dev)
        pool_out = (torch.empty(cfg.batch, pool_cap, dtype=torch.int32, device=dev),
                    torch.empty(cfg.batch, dtype=torch.int32, device=dev))
        sel_out = (torch.empty(cfg.batch, HSI_TOP_K, dtype=torch.int32, device=dev),
                   torch.empty(cfg.batch, dtype=torch.int32, device=dev))
        hsi_ws = torch.empty(kvq.kv_hsi_candidates(None, cfg.batch, T, None, HSI_BLOCK, HSI_TOP_BLOCKS, None, None,
                                                   None, 0), dtype=torch.uint8, device=dev)
        sp_ws = torch.zeros(kvq.kv_decode_attention_sparse(cache.struct, None, kvq.DT_BF16, cfg.hq, None, None,
                                                           HSI_TOP_K, 1.0, None, None, 0,
                                                           kvq.KVDecodeOpts(args.splits, None, None, 1)),
                            dtype=torch.uint8, device=dev)

    def step(i=None):
        cache.append(k_new, v_new, T - n_new)
        if args.hsi:
            pool, pool_n = hsi_candidates(full_scores, lens, HSI_BLOCK, HSI_TOP_BLOCKS, out=pool_out, ws=hsi_ws)
            sel, sel_n = hsi_select(pool_scores, pool, pool_n, HSI_TOP_K, out=sel_out)
            cache.decode_sparse(q, sel, sel_n, scale, splits=args.splits, out=out, ws=sp_ws,
                                events=None if i is None else ev[i])
            return
        cache.decode(q, lens, scale, splits=args.splits, out=out, ws=ws,
                     events=None if i is None else ev[i])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # eager timed pass: events around the split-context attention kernel
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    s0.record()
    for i in range(args.steps):
        step(i)
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_eager = s0.elapsed_time(s1) / args.steps
    dec_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    ms_step = ms_eager
    if not args.no_graph:
        # The same step captured once as a HIP graph and replayed: the launch
        # overhead of the four kernels leaves the timed region.  Every replay must
        # reproduce the eager output bit for bit, with eager steps in between.
        ref = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref):
                raise RuntimeError("graph replay differs from the eager step")
            step()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        s0.record()
        for _ in range(args.steps):
            graph.replay()
        s1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_step = s0.elapsed_time(s1) / args.steps
    nbytes = counted_bytes(cfg, cache.layout, kvq, args.sink, args.recent)
    if args.hsi:
        # the step reads the full-mode scores, the pool's scores and the packed
        # bytes of the selected positions
        n_sel = int(sel_out[1].sum())
        nbytes = 4 * cfg.batch * (T + pool_cap) + kvq.kv_bytes_per_token(cache.layout, 1) * n_sel
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (dec_ms * 1e-3) / 1e9
    res = {
        "metric": "decode-attn KV GB/s read (% of HBM peak) + query-tokens/s at fixed context",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "format": cfg.fmt, "batch": cfg.batch, "q_heads": cfg.hq,
                   "kv_heads": cfg.hkv, "head_dim": cfg.head_dim, "rope_dim": cfg.rope_dim,
                   "context": T, "counted_bytes_per_step": nbytes,
                   "splits": args.splits or "auto", "queries_per_seq": nq,
                   "bf16_sink_tokens": args.sink, "bf16_recent_tokens": args.recent,
                   **({"page_tokens": args.page_tokens} if args.page_tokens else {}),
                   **({"rotation": args.rotation} if cfg.fmt == "turbo" else {})},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "query_tokens_per_s": round(nq * cfg.batch / (ms_step * 1e-3), 1),
        "wall_s": round(wall, 3),
        "timing": "hip-graph replay of the step" if not args.no_graph else "eager launches",
        "ms_per_step_eager": round(ms_eager, 5),
        "roofline": roofline(cfg, nbytes, dec_ms, nq, bool(args.sink or args.recent), bool(args.page_tokens)),
    }
    if args.hsi:
        # the dominant kernel is the sparse decode on the general (fp32 vector) kernel:
        # per selected position and query head, key_width + head_dim multiply-adds
        # (the latent cache's gather kernel runs them on the fp16 matrix cores); the
        # FP4 / QJL / TurboQuant gather kernels are priced by the packed bytes they
        # gather, the general kernel (KIVI-2) against the fp32 vector peak
        res["metric"] = "HSI sparse decode step: bytes read GB/s + query-tokens/s at fixed context"
        res["config"].update(hsi={"block": HSI_BLOCK, "top_blocks": HSI_TOP_BLOCKS, "top_k": HSI_TOP_K,
                                  "selected_positions": n_sel})
        if cfg.fmt in ("fp4", "qjl1", "turbo"):
            gathered = kvq.kv_bytes_per_token(cache.layout, 1) * n_sel
            ach = gathered / (dec_ms * 1e-3) / 1e9
            res["roofline"] = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                               "kernel": "sparse split-context attention", "kernel_us": round(dec_ms * 1e3, 2)}
        else:
            flops = 2.0 * cfg.hq * n_sel * (cfg.key_width + cfg.head_dim)
            ach = flops / (dec_ms * 1e-3) / 1e12
            mfma = cfg.fmt == "latent"
            peak = MFMA_F16_PEAK_TFLOPS if mfma else FP32_VALU_PEAK_TFLOPS
            res["roofline"] = {"bound": "mfma" if mfma else "alu", "achieved": round(ach, 2), "peak": peak,
                               "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": None,
                               "kernel": "sparse split-context attention", "kernel_us": round(dec_ms * 1e3, 2)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, rotation=args.rotation if cfg.fmt == "turbo" else "haar",
                                           hsi=args.hsi)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
