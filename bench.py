"""Decode-attention bandwidth benchmark for the packed low-bit KV cache.

One step = the whole hot path for one decode token of every sequence: append
that token's K/V into the packed cache (the format's pack kernel) and run
single-query attention over the full context (query prep, split-context
attention, merge), at a fixed context length.

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

HBM_PEAK_GBS = 8000.0


def counted_bytes(cfg, lib_layout, kvq):
    """Packed KV + scales/norms read by one decode step over cfg.context tokens."""
    per_tok = kvq.kv_bytes_per_token(lib_layout, 1)
    return per_tok * cfg.batch * cfg.context


def cpu_baseline(cfg, budget_s=12.0):
    """Time the oracle's decode on a bounded sample: one (sequence, KV head) unit at a time."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import attention as OA
    from oracle import formats as OF
    from oracle.bytes import per_token_head

    if cfg.fmt != "fp4":
        return None
    T = cfg.context
    unit = cfg.scaled(batch=1, hkv=1, hq=cfg.group)
    K, V = synth.make_kv(unit, device="cpu")
    enc = OF.encode_cache("fp4", K.float().numpy().astype(np.float64), V.float().numpy().astype(np.float64))
    q = synth.make_queries(unit, device="cpu").float().numpy().astype(np.float64)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    units = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            OA.decode_attention("fp4", enc, q, [T], scale, 1)
            units += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    nbytes = units * T * per_token_head("fp4", cfg.head_dim)
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{units} x decode of 1 sequence x 1 KV head ({cfg.group} q heads) over {T} tokens, "
                      f"fp64 numpy, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="fp4_b16_t32k")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
                                synth.gaussian_matrix(cfg.seed, 128, cfg.head_dim, stream=2))
    cache = PackedKVCache(cfg.fmt, cfg.batch, cfg.hkv, cfg.head_dim, cfg.context, cfg.rope_dim, device=dev,
                          constants=consts)
    T = cfg.context
    # prefill T-1 tokens (untimed), one sequence and 16K tokens at a time to bound input memory
    for b in range(cfg.batch):
        seq = cache.sequence(b)
        for t0 in range(0, T - 1, 16384):
            t1 = min(T - 1, t0 + 16384)
            if cfg.fmt == "latent":
                seq.append(synth.make_latent(cfg, b, b + 1, t0, t1, device=dev), None, t0)
            else:
                K, V = synth.make_kv(cfg, b, b + 1, t0, t1, device=dev)
                seq.append(K, V, t0)
    # the decode token's K/V (appended at T-1 inside every step)
    if cfg.fmt == "latent":
        k_new, v_new = synth.make_latent(cfg, 0, cfg.batch, T - 1, T, device=dev), None
    else:
        k_new, v_new = synth.make_kv(cfg, 0, cfg.batch, T - 1, T, device=dev)
    q = synth.make_queries(cfg, device=dev)
    lens = torch.full((cfg.batch,), T, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(cfg.key_width)
    out = torch.empty(cfg.batch, cfg.hq, cfg.head_dim, dtype=torch.float32, device=dev)
    ws = torch.zeros(cache.workspace_bytes(cfg.hq, T, args.splits, q.dtype), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:  # torch creates the HIP event on first record; the library records it afterwards
        a.record()
        b.record()

    def step(i=None):
        cache.append(k_new, v_new, T - 1)
        cache.decode(q, lens, scale, splits=args.splits, out=out, ws=ws,
                     events=None if i is None else ev[i])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    s0.record()
    for i in range(args.steps):
        step(i)
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = s0.elapsed_time(s1) / args.steps
    dec_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    nbytes = counted_bytes(cfg, cache.layout, kvq)
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
                   "splits": args.splits or "auto"},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "query_tokens_per_s": round(cfg.batch / (ms_step * 1e-3), 1),
        "wall_s": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_split_kernel", "kernel_us": round(dec_ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
