"""Decode-attention bandwidth benchmark for the packed low-bit KV cache.

One step = the whole hot path for one decode token of every sequence: append
that token's K/V into the packed cache (the format's pack kernel; the 1M-context
workload appends 32,768 tokens in bulk) and run attention over the full context
(query prep, split-context attention, merge), at a fixed context length.

With no --config the bench runs all five workloads and prints ONE JSON line:
the headline fields are those of the largest single-GPU workload,
latent_b64_t64k (1.88 GB of packed cache read per step), and `workloads` holds
one record per workload (step time median and min, GB/s, % of HBM peak, query
tokens/s, the attention kernel's roofline, the CPU oracle baseline).

Timing, per workload:
  * inputs are resident in HBM before anything is timed;
  * before every timed step a streaming read of a separate 1 GiB buffer
    (outside the event pair) evicts the 256 MB MALL and the L2s, so each step
    reads its cache from HBM;
  * the step is captured once as a HIP graph (checked bit for bit against the
    eager step) and replayed; each replay is bracketed by its own HIP events on
    the stream it runs on; median and min are reported;
  * the attention kernel's own duration (for the roofline) comes from HIP
    events the library records immediately around its launch, in an eager pass
    over the same number of flushed steps.
A plain streaming-read kernel (kvq_probe.h) is timed the same way over 1 GiB:
the bandwidth a kernel that only reads reaches on this part, for context.  Two
more reference kernels (kvq_probe.h), a loop of 32x32x16 fp16 matrix products
and a loop of LDS reads, one workgroup of 4 waves per compute unit, give the
compute and LDS rates the part delivers as clocked under such load; the latent
record carries its kernel's fraction of the first and the time its LDS reads
alone would take at the second (`measured_ceilings`).

`value` is decode KV GB/s: the packed bytes the attention reads per step
(codes + scales/norms of every cached token) over the median step time.
"""

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_VALU_PEAK_TFLOPS = 157.3  # fp32 vector peak (256 CUs, 2.4 GHz)
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 matrix-core peak
HBM_PEAK_GBS = 8000.0
ALL_WORKLOADS = ["kivi2_tiny", "fp4_b16_t32k", "turbo_b8_t128k", "qjl1_b1_t1m", "latent_b64_t64k"]
HEADLINE = "latent_b64_t64k"  # the largest single-GPU workload by bytes read per step
FLUSH_BYTES = 1 << 30         # 4x the 256 MB MALL
CPU_SAMPLE_TOKENS = 131072    # context of the CPU oracle's decode sample (whole context if shorter)

# the arithmetic each workload's attention kernel computes in
DTYPE = {
    "kivi2": "fp16 MFMA operands (codes exact, query x scale as an fp16 pair, values rounded once), fp32 accumulate and softmax",
    "fp4": "fp16 MFMA operands (E2M1 x bf16 scale exact), fp32 accumulate and softmax",
    "turbo": "fp4 x fp6 and fp16 MFMA operands, fp32 accumulate and softmax",
    "qjl1": "fp4 x fp8 and fp16 MFMA operands, fp32 accumulate and softmax",
    "latent": "fp16 / bf16 MFMA operands (E2M1 x bf16 scale exact), fp32 accumulate and softmax",
}


def counted_bytes(cfg, lib_layout, kvq, sink=0, recent=0):
    """Packed KV + scales/norms read by one decode step over cfg.context tokens
    (with bf16 sink / recent windows: those tokens as bf16 K and V instead)."""
    per_tok = kvq.kv_bytes_per_token(lib_layout, 1)
    window = min(cfg.context, sink + recent)
    return (per_tok * cfg.batch * (cfg.context - window)
            + cfg.batch * cfg.hkv * window * cfg.head_dim * 2 * 2)


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0)), os.cpu_count()


def cpu_baseline(cfg, budget_s=2.5, rotation="haar", hsi=False):
    """The oracle as it stands, on a bounded sample of the workload: one
    (sequence, KV head) unit (with its query-head group) over the first
    min(context, CPU_SAMPLE_TOKENS) tokens.  Encode (the oracle's append) of the
    sample is timed once; decode (or, with hsi, the oracle's candidate pool,
    reindex top-k and sparse decode) is repeated for about budget_s seconds.
    BLAS runs on every core this process may use."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import attention as OA
    from oracle import formats as OF
    from oracle.bytes import per_token_head
    from oracle.lloyd_max import canonical_codebook
    from oracle.rotation import canonical_hadamard_rotation, canonical_projection, canonical_rotation

    model, cores, ncpu = cpu_info()
    T = min(cfg.context, CPU_SAMPLE_TOKENS)
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
    with threadpool_limits(limits=cores):
        inputs = []
        for t0 in range(0, T, 65536):
            t1 = min(T, t0 + 65536)
            if cfg.fmt == "latent":
                inputs.append(synth.make_latent(unit, 0, 1, t0, t1, device="cpu").float().numpy().astype(np.float64))
            else:
                K, V = synth.make_kv(unit, 0, 1, t0, t1, device="cpu")
                inputs.append((K.float().numpy().astype(np.float64), V.float().numpy().astype(np.float64)))
        te = time.perf_counter()
        parts = []
        for x in inputs:
            if cfg.fmt == "latent":
                parts.append(OF.encode_cache("latent", latent=x, latent_dim=cfg.head_dim))
            else:
                parts.append(OF.encode_cache(cfg.fmt, x[0], x[1], consts=consts))
        enc_s = time.perf_counter() - te
        axis = 1 if cfg.fmt == "latent" else 2
        enc = {k: np.concatenate([e[k] for e in parts], axis=axis) for k in parts[0]}
        q = synth.make_queries(unit, device="cpu").float().numpy().astype(np.float64)
        scale = 1.0 / math.sqrt(cfg.key_width)
        if hsi:
            from oracle.hsi import candidate_pool, decode_attention_sparse, select_top_k
            full = synth.make_indexer_scores(cfg.seed, 1, T).numpy()[0]
            pool_scores = synth.make_indexer_scores(cfg.seed, 1, 8 * 2048, layer=1).numpy()[0]
        units = 0
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
    pth = per_token_head(cfg.fmt, cfg.head_dim, cfg.rope_dim)
    base = {"unit": "GB/s", "cores": cores, "kind": "oracle", "cpu_model": model, "cpu_count": ncpu,
            "encode_value": round(T * pth / enc_s / 1e9, 6), "encode_unit": "GB/s of packed cache written",
            "encode_tokens_per_s": round(T / enc_s, 1),
            "encode_sample": f"oracle append of {T} tokens of 1 sequence x 1 KV head, {enc_s:.2f} s"}
    what = "HSI pool + top-512 + sparse decode" if hsi else "decode"
    if hsi:
        nbytes = units * (4 * (T + 8 * 2048) + 512 * pth)
    else:
        nbytes = units * T * pth
    base.update(value=round(nbytes / el / 1e9, 6),
                sample=f"{units} x {what} of 1 sequence x 1 KV head ({unit.hq} q heads) over {T} tokens "
                       f"(workload context {cfg.context}), fp64 numpy, BLAS on {cores} threads, {el:.1f} s")
    return base


def measured_profile(workload, kind):
    """Fields of the committed counter summary profiles/*_<workload>_<kind>.txt
    for the attention kernel, or None when there is none or the kernel's source
    has changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_{kind}.txt"))):
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        src = os.path.join(ROOT, kv.get("source", ""))
        if kv.get("role", "attention") != "attention" or not os.path.isfile(src):
            continue
        if hashlib.sha256(open(src, "rb").read()).hexdigest() == kv.get("source_sha256"):
            return kv
    return None


def roofline(cfg, nbytes, kern_us, nq=1, plain=True):
    """Roofline of the split-context attention kernel from its event-timed duration.
    The counter summaries cover the one-query, contiguous, window-free kernels."""
    pmc = measured_profile(cfg.name, "pmc") if plain and nq == 1 else None
    util = measured_profile(cfg.name, "util") if plain and nq == 1 else None
    traffic = int(pmc["traffic_bytes_per_launch"]) if pmc and "traffic_bytes_per_launch" in pmc else None
    sec = kern_us * 1e-6
    if cfg.fmt == "latent":
        # 128 heads x (576 + 512) x 2 flop per token: a dense contraction on fp16 matrix cores
        flops = 2.0 * nq * cfg.batch * cfg.context * cfg.hq * (cfg.key_width + cfg.head_dim)
        ach = flops / sec / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
             "hbm_gbs": round(nbytes / sec / 1e9, 2)}
    else:
        ach = nbytes / sec / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
    r.update(kernel="split-context attention", kernel_us=round(kern_us, 2),
             algorithmic_bytes_per_launch=nbytes)
    if util:
        r["utilisation"] = {k: float(util[k]) for k in ("mfma_busy", "valu_active", "lds_active", "wait_inst_share")
                            if k in util}
    return r


class Flusher:
    """Evicts the MALL and the L2s before a timed launch: a streaming read of a
    1 GiB buffer (a read, so that the lines it leaves are clean: a copy would
    leave dirty lines whose write-back then lands inside the timed kernel)."""

    def __init__(self, torch, kvq, dev, nbytes):
        self.kvq = kvq
        self.torch = torch
        self.buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev) if nbytes else None
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def __call__(self):
        if self.buf is not None:
            self.kvq.kv_stream_read(self.buf.data_ptr(), self.buf.numel() * 4, self.sink.data_ptr(),
                                    self.torch.cuda.current_stream().cuda_stream)


def timed(torch, fn, n, flush):
    """Run fn n times, each flushed first and bracketed by its own events on the
    current stream; returns the per-call milliseconds."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        flush()
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def stream_read_reference(torch, kvq, dev, flush, steps):
    buf = torch.full((FLUSH_BYTES // 4,), 7, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        kvq.kv_stream_read(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), st)
    ms = timed(torch, lambda i: kvq.kv_stream_read(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), st),
               max(steps, 10), flush)
    med = statistics.median(ms)
    gbs = buf.numel() * 4 / (med * 1e-3) / 1e9
    return {"kernel": "stream_read_kernel (16-byte loads, 8 in flight per thread, a contiguous run per workgroup)", "bytes": buf.numel() * 4,
            "us_median": round(med * 1e3, 2), "us_min": round(min(ms) * 1e3, 2), "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def compute_references(torch, kvq, dev, steps):
    """Median rates of the matrix-core and LDS reference kernels (kvq_probe.h),
    256 workgroups of 4 waves (one wave per SIMD, as in the latent decode)."""
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    blocks, it_mfma, it_lds = 256, 2048, 2048
    flop = blocks * 4 * it_mfma * 8 * 32768.0
    lds_bytes = blocks * 4 * it_lds * 8 * 1024.0
    for _ in range(3):
        kvq.kv_mfma_probe(blocks, it_mfma, sink.data_ptr(), st)
        kvq.kv_lds_probe(blocks, it_lds, sink.data_ptr(), st)
    n = max(steps, 10)
    ms_m = timed(torch, lambda i: kvq.kv_mfma_probe(blocks, it_mfma, sink.data_ptr(), st), n, lambda: None)
    ms_l = timed(torch, lambda i: kvq.kv_lds_probe(blocks, it_lds, sink.data_ptr(), st), n, lambda: None)
    tflops = flop / (statistics.median(ms_m) * 1e-3) / 1e12
    lds_tbs = lds_bytes / (statistics.median(ms_l) * 1e-3) / 1e12
    return {"mfma_kernel": "mfma_probe_kernel (v_mfma_f32_32x32x16_f16, 2 chains, operands in registers)",
            "mfma_tflops": round(tflops, 1), "mfma_frac_of_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "lds_kernel": "lds_probe_kernel (ds_read_b128, 1 KiB per wave and read, conflict-free)",
            "lds_tbs": round(lds_tbs, 2)}


def latent_lds_bytes(cfg, nq=1):
    """LDS bytes the latent decode reads per launch: each of a workgroup's 4
    waves reads the whole dequantised 32-token tile, its keys (576 fp16/bf16
    channels) for S = K Q^T and its values (512 channels, transposed) for P V."""
    tiles = nq * cfg.batch * cfg.context / 32
    return tiles * 4 * 32 * (cfg.key_width + cfg.head_dim) * 2


def run_workload(name, args, dev, flush, cpu):
    import torch

    import synth
    from bit_kv_cache_04_amd import kvq
    from bit_kv_cache_04_amd.cache import PackedKVCache, make_constants

    cfg = synth.CONFIGS[name]
    ov = {k: v for k, v in (("batch", args.batch), ("context", args.context), ("hq", args.q_heads),
                            ("hkv", args.kv_heads), ("head_dim", args.head_dim)) if v}
    if ov:  # a resized copy of the workload: its own name, so no committed counter summary applies
        cfg = cfg.scaled(name=name + "@" + ",".join(f"{k}={v}" for k, v in ov.items()), **ov)
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
    rot_kind = {}
    if cfg.fmt == "turbo" and args.butterfly:
        # the structured rotation applied as a butterfly: no dense matrix at all
        rot_kind = dict(rotation=kvq.ROT_HADAMARD_BITREV if args.rotation == "hadamard" else kvq.ROT_HADAMARD)
        consts.pop("rot")
    cache = PackedKVCache(cfg.fmt, cfg.batch, cfg.hkv, cfg.head_dim, cfg.context, cfg.rope_dim, device=dev,
                          constants=consts, sink_tokens=args.sink, recent_tokens=args.recent, **paging, **rot_kind)
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

    steps = args.steps
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for evs in (kev, aev):
        for a, b in evs:  # torch creates the HIP event on first record; the library records it afterwards
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
        if i is not None:
            aev[i][0].record()
        cache.append(k_new, v_new, T - n_new)
        if i is not None:
            aev[i][1].record()
        if args.hsi:
            pool, pool_n = hsi_candidates(full_scores, lens, HSI_BLOCK, HSI_TOP_BLOCKS, out=pool_out, ws=hsi_ws)
            sel, sel_n = hsi_select(pool_scores, pool, pool_n, HSI_TOP_K, out=sel_out)
            cache.decode_sparse(q, sel, sel_n, scale, splits=args.splits, out=out, ws=sp_ws,
                                events=None if i is None else kev[i])
            return
        cache.decode(q, lens, scale, splits=args.splits, out=out, ws=ws, events=None if i is None else kev[i])

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    # eager pass: events around the split-context attention kernel and the append
    w0 = time.perf_counter()
    eager_ms = timed(torch, step, steps, flush)
    wall = time.perf_counter() - w0
    kern_ms = [a.elapsed_time(b) for a, b in kev]
    app_ms = [a.elapsed_time(b) for a, b in aev]
    step_ms = eager_ms
    if not args.no_graph:
        # The same step captured once as a HIP graph and replayed: the launch
        # overhead of the step's kernels leaves the timed region.  Every replay must
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
                raise RuntimeError(f"{name}: graph replay differs from the eager step")
            step()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            flush()
            graph.replay()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        step_ms = timed(torch, lambda i: graph.replay(), steps, flush)
        wall = time.perf_counter() - w0
    ms_med, ms_min = statistics.median(step_ms), min(step_ms)
    kern_us = statistics.median(kern_ms) * 1e3
    nbytes = counted_bytes(cfg, cache.layout, kvq, args.sink, args.recent)
    if args.hsi:
        # the step reads the full-mode scores, the pool's scores and the packed
        # bytes of the selected positions
        n_sel = int(sel_out[1].sum())
        nbytes = 4 * cfg.batch * (T + pool_cap) + kvq.kv_bytes_per_token(cache.layout, 1) * n_sel
    gbs = nbytes / (ms_med * 1e-3) / 1e9
    plain = not (args.sink or args.recent or args.page_tokens or args.hsi)
    rec = {
        "workload": cfg.name,
        "config": {"workload": cfg.name, "format": cfg.fmt, "batch": cfg.batch, "q_heads": cfg.hq,
                   "kv_heads": cfg.hkv, "head_dim": cfg.head_dim, "rope_dim": cfg.rope_dim,
                   "context": T, "appended_per_step": n_new, "counted_bytes_per_step": nbytes,
                   "splits": args.splits or "auto", "queries_per_seq": nq,
                   "bf16_sink_tokens": args.sink, "bf16_recent_tokens": args.recent,
                   **({"page_tokens": args.page_tokens} if args.page_tokens else {}),
                   **({"rotation": args.rotation} if cfg.fmt == "turbo" else {})},
        "dtype": DTYPE[cfg.fmt],
        "value": round(gbs, 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_med, 5),
        "ms_per_step_min": round(ms_min, 5),
        "ms_per_step_eager": round(statistics.median(eager_ms), 5),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "query_tokens_per_s": round(nq * cfg.batch / (ms_med * 1e-3), 1),
        "wall_s": round(wall, 3),
        "timing": ("hip-graph replay of the step" if not args.no_graph else "eager launches")
                  + ", median of per-step HIP events, MALL flushed before each step",
        "roofline": roofline(cfg, nbytes, kern_us, nq, plain),
        "attention_kernel_us_min": round(min(kern_ms) * 1e3, 2),
        "append_us": round(statistics.median(app_ms) * 1e3, 2),
    }
    if cfg.append_new:
        # bulk append: bf16 K and V in, packed rows out (QJL keys 18 B + FP4 values 80 B per token-head)
        rows = cfg.batch * cfg.hkv * n_new
        io = 2 * rows * cfg.head_dim * 2 + rows * kvq.kv_bytes_per_token(cache.layout, 1) // cfg.hkv
        a_us = statistics.median(app_ms) * 1e3
        rec["append_roofline"] = {"bound": "hbm", "achieved": round(io / (a_us * 1e-6) / 1e9, 2),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(io / (a_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                  "kernel": "bulk append", "kernel_us": round(a_us, 2),
                                  "algorithmic_bytes_per_launch": io}
    if args.hsi:
        rec["metric"] = "HSI sparse decode step: bytes read GB/s + query-tokens/s at fixed context"
        rec["config"].update(hsi={"block": HSI_BLOCK, "top_blocks": HSI_TOP_BLOCKS, "top_k": HSI_TOP_K,
                                  "selected_positions": n_sel})
        if cfg.fmt in ("fp4", "qjl1", "turbo"):
            gathered = kvq.kv_bytes_per_token(cache.layout, 1) * n_sel
            ach = gathered / (kern_us * 1e-6) / 1e9
            rec["roofline"] = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                               "kernel": "sparse split-context attention", "kernel_us": round(kern_us, 2)}
        else:
            # per selected position and query head, key_width + head_dim multiply-adds
            # (the latent cache's gather kernel runs them on the fp16 matrix cores,
            # KIVI-2 on the general fp32 vector kernel)
            flops = 2.0 * cfg.hq * n_sel * (cfg.key_width + cfg.head_dim)
            ach = flops / (kern_us * 1e-6) / 1e12
            mfma = cfg.fmt == "latent"
            peak = MFMA_F16_PEAK_TFLOPS if mfma else FP32_VALU_PEAK_TFLOPS
            rec["roofline"] = {"bound": "mfma" if mfma else "alu", "achieved": round(ach, 2), "peak": peak,
                               "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": None,
                               "kernel": "sparse split-context attention", "kernel_us": round(kern_us, 2)}
    rec["_cfg"] = cfg
    if not args.no_graph:
        del graph
    del cache, ws, out, k_new, v_new, q
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None,
                    help="one workload; default: all five, with latent_b64_t64k as the headline")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--batch", type=int, default=0, help="resize the workload: sequences")
    ap.add_argument("--context", type=int, default=0, help="resize the workload: cached tokens per sequence")
    ap.add_argument("--q-heads", type=int, default=0, help="resize the workload: query heads")
    ap.add_argument("--kv-heads", type=int, default=0, help="resize the workload: KV heads")
    ap.add_argument("--head-dim", type=int, default=0, help="resize the workload: head dimension")
    ap.add_argument("--sink", type=int, default=0, help="leading tokens kept bf16 (per-head formats)")
    ap.add_argument("--recent", type=int, default=0, help="trailing tokens kept bf16 (per-head formats)")
    ap.add_argument("--queries", type=int, default=1,
                    help="query tokens per sequence (drafted positions checked in one pass); the step "
                         "appends that many tokens")
    ap.add_argument("--butterfly", action="store_true",
                    help="with --rotation hadamard / hadamard_plain: apply R as a Hadamard butterfly "
                         "(layout.rotation) instead of a dense matrix")
    ap.add_argument("--rotation", default="haar", choices=["haar", "hadamard", "hadamard_plain"],
                    help="TurboQuant rotation: a Haar draw, or the Hadamard transform with (or without) "
                         "the bit-reversal permutation")
    ap.add_argument("--page-tokens", type=int, default=0,
                    help="paged storage: tokens per page, the pool's pages assigned to sequences in a seeded "
                         "shuffled order")
    ap.add_argument("--hsi", action="store_true",
                    help="hierarchical sparse indexing: candidate pool (top 2048 blocks of 8 by synthetic full-mode "
                         "scores), reindex top 512 (synthetic pool scores), decode over the selected positions")
    ap.add_argument("--no-flush", action="store_true", help="do not evict the MALL before each timed step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph replay")
    args = ap.parse_args()
    if args.butterfly and args.rotation == "haar":
        ap.error("--butterfly needs --rotation hadamard or hadamard_plain (a Haar rotation has no butterfly)")
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode shards by sequence and KV head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_kv_cache_04_amd import kvq

    dev = torch.device("cuda:0")
    flush = Flusher(torch, kvq, dev, 0 if args.no_flush else FLUSH_BYTES)
    names = [args.config] if args.config else ALL_WORKLOADS
    headline = args.config or HEADLINE
    records = {}
    for name in names:
        print(f"bench: {name} ...", file=sys.stderr, flush=True)
        records[name] = run_workload(name, args, dev, flush, not args.no_cpu_baseline)
    ref = stream_read_reference(torch, kvq, dev, flush, args.steps)
    cref = compute_references(torch, kvq, dev, args.steps)
    for name, rec in records.items():
        cfg = rec.get("_cfg")
        if cfg is not None and cfg.fmt == "latent" and rec["roofline"].get("bound") == "mfma":
            r = rec["roofline"]
            lds = latent_lds_bytes(cfg, rec["config"].get("queries_per_seq", 1))
            r["measured_ceilings"] = {
                "mfma_tflops": cref["mfma_tflops"],
                "frac_of_measured_mfma": round(r["achieved"] / cref["mfma_tflops"], 4),
                "mfma_floor_us": round(r["achieved"] * r["kernel_us"] / cref["mfma_tflops"], 1),
                "lds_bytes_per_launch": int(lds),
                "lds_tbs": cref["lds_tbs"],
                "lds_floor_us": round(lds / (cref["lds_tbs"] * 1e12) * 1e6, 1)}
    if not args.no_cpu_baseline:
        for name in names:
            cfg = records[name].pop("_cfg")
            print(f"bench: cpu baseline {name} ...", file=sys.stderr, flush=True)
            records[name]["cpu_baseline"] = cpu_baseline(
                cfg, rotation=args.rotation if cfg.fmt == "turbo" else "haar", hsi=args.hsi)
    h = records[headline]
    res = {
        "metric": h.get("metric", "decode-attn KV GB/s read (% of HBM peak) + query-tokens/s at fixed context"),
        "value": h["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "ms_per_step_min": h["ms_per_step_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic (seeded N(0,1) K/V/latent/queries, key outlier channels; no dataset or weights)",
        "config": h["config"],
        "pct_hbm_peak": h["pct_hbm_peak"],
        "query_tokens_per_s": h["query_tokens_per_s"],
        "timing": h["timing"],
        "roofline": h["roofline"],
        "stream_read_reference": ref,
        "compute_reference": cref,
        "workloads": {n: {k: v for k, v in r.items() if k not in ("workload", "_cfg")} for n, r in records.items()},
    }
    if "cpu_baseline" in h:
        res["cpu_baseline"] = h["cpu_baseline"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
