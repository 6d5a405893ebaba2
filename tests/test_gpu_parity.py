"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Packed bytes must be bit-exact (KIVI-2 and FP4 by definition; TurboQuant and
QJL sketches are computed so that they match the exact-arithmetic signs and
codes, and any difference is counted against the 1e-5 tie budget); attention
outputs must be within 2e-3 max relative error per (sequence, query head) row.
Small shapes span several 32-token tiles, several splits and a ragged tail.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import (RTOL, assert_bytes_equal, gpu_buffers, host64, inputs, new_cache, oracle_constants,
                         oracle_encode, row_rel_err, softmax_scale)
from bit_kv_cache_04_amd import kvq
from oracle import attention as OA

pytestmark = pytest.mark.gpu

C = synth.CONFIGS
SMALL = {
    "kivi2": C["kivi2_tiny"],
    "fp4": C["fp4_b16_t32k"].scaled(batch=2, hq=8, hkv=2, context=1000),
    "turbo": C["turbo_b8_t128k"].scaled(batch=2, hq=16, hkv=2, context=777),
    "qjl1": C["qjl1_b1_t1m"].scaled(batch=2, hq=8, hkv=2, context=1500),
    "latent": C["latent_b64_t64k"].scaled(batch=2, hq=128, context=300),
}


def _build(cfg, chunks=2, ramp=None):
    """Cache of cfg's seeded inputs; ramp multiplies token t's key (latent) by 1 + ramp * t / T."""
    torch.manual_seed(0)
    cache = new_cache(cfg)
    K, V = inputs(cfg)
    T = cfg.context
    if ramp is not None:
        r = 1.0 + ramp * torch.arange(T, device=K.device, dtype=torch.float32) / T
        r = r.view(1, T, 1) if cfg.fmt == "latent" else r.view(1, 1, T, 1)
        K = (K.float() * r).to(K.dtype)
    step = -(-T // chunks)
    if cfg.fmt == "kivi2":
        step = -(-step // 32) * 32
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        if cfg.fmt == "latent":
            cache.append(K[:, t0:t1].contiguous(), None, t0)
        else:
            cache.append(K[:, :, t0:t1].contiguous(), V[:, :, t0:t1].contiguous(), t0)
    torch.cuda.synchronize()
    return cache, K, V


@pytest.mark.parametrize("fmt", list(SMALL))
def test_append_bytes_match_oracle(fmt):
    cfg = SMALL[fmt]
    print(f"[append] {fmt} {cfg}", flush=True)
    cache, K, V = _build(cfg)
    want = oracle_encode(cfg, host64(K), host64(V), oracle_constants(cfg))
    assert_bytes_equal(gpu_buffers(cache), want, fmt)


@pytest.mark.parametrize("fmt", list(SMALL))
def test_decode_matches_oracle(fmt):
    cfg = SMALL[fmt]
    print(f"[decode] {fmt} {cfg}", flush=True)
    cache, K, V = _build(cfg)
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V), consts)
    q = synth.make_queries(cfg, device="cuda")
    lens = synth.seq_lens_for(cfg, ragged=True)
    lens[-1] = 1                                        # a single-token context
    lens_d = torch.from_numpy(lens).cuda()
    out = cache.decode(q, lens_d, softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention(cfg.fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, consts,
                              latent_dim=cfg.head_dim)
    err = row_rel_err(out, ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _bf16_step(x, up):
    """The bf16 neighbour of bf16 x (x != 0) one unit further from (up) or nearer to zero."""
    u = np.array([x], np.float32).view(np.uint32)
    u = u + np.uint32(0x10000) if up else u - np.uint32(0x10000)
    return float(u.view(np.float32)[0])


def _fp4_edge_groups(rng, n_groups):
    """bf16-exact 16-value groups at the FP4 encoder's decision edges.

    Each group's absmax A fixes s = bf16(A / 6); the other values are exact
    midpoints t * s between E2M1 neighbours (where bf16 holds them), their bf16
    neighbours, zeros and signed zeros.  Exponents span ordinary magnitudes,
    both ends of [2^-100, 2^100] and beyond them on either side.
    """
    from oracle.numerics import round_bf16
    exps = [(-6, 7)] * 6 + [(-112, -104), (104, 112)]
    out = np.zeros((n_groups, 16))
    for gi in range(n_groups):
        kind = gi % 10
        if kind == 9:
            continue  # an all-zero group
        if kind == 8:
            a = float(2.0 ** rng.choice([-100, 100]))
        else:
            lo, hi = exps[kind]
            a = float(round_bf16(rng.uniform(1.0, 2.0) * 2.0 ** int(rng.integers(lo, hi))))
        s = float(round_bf16(a / 6.0))
        cands = [0.0]
        for t in E2M1_MIDPOINTS:
            x = t * s
            if float(round_bf16(x)) == x:
                cands += [x, _bf16_step(x, True), _bf16_step(x, False)]
        vals = rng.choice(np.array(cands), 15) * rng.choice([-1.0, 1.0], 15)
        g = np.concatenate([[a * rng.choice([-1.0, 1.0])], vals])
        out[gi] = g[rng.permutation(16)]
    return out


@pytest.mark.parametrize("fmt", ["fp4", "qjl1", "latent"])
def test_fp4_encoder_decision_edges(fmt):
    """FP4 codes and scales at exact midpoints, their neighbours, saturation,
    signed zeros and extreme exponents equal the oracle's, byte for byte."""
    cfg = SMALL[fmt].scaled(batch=1, context=96)
    print(f"[fp4 edges] {fmt}", flush=True)
    rng = np.random.default_rng(11)
    T = cfg.context
    if fmt == "latent":
        K = _fp4_edge_groups(rng, T * (cfg.head_dim + cfg.rope_dim) // 16).reshape(1, T, -1)
        V = None
    else:
        V = _fp4_edge_groups(rng, cfg.hkv * T * cfg.head_dim // 16).reshape(1, cfg.hkv, T, cfg.head_dim)
        if fmt == "fp4":
            K = _fp4_edge_groups(rng, cfg.hkv * T * cfg.head_dim // 16).reshape(V.shape)
        else:
            K = rng.standard_normal(V.shape)
    dev = lambda a: torch.from_numpy(a).to(torch.float32).to(torch.bfloat16).cuda() if a is not None else None
    Kd, Vd = dev(K), dev(V)
    cache = new_cache(cfg)
    cache.append(Kd, Vd, 0)
    torch.cuda.synchronize()
    want = oracle_encode(cfg, host64(Kd), host64(Vd), oracle_constants(cfg))
    assert_bytes_equal(gpu_buffers(cache), want, f"{fmt} decision edges")


@pytest.mark.parametrize("fmt", ["fp4", "turbo", "qjl1", "latent"])
def test_token_by_token_append_equals_bulk(fmt):
    """A decode loop appends one token per step; the bytes must equal a bulk append."""
    cfg = SMALL[fmt].scaled(context=70)
    bulk, K, V = _build(cfg, chunks=1)
    step = new_cache(cfg)
    for t in range(cfg.context):
        if fmt == "latent":
            step.append(K[:, t:t + 1].contiguous(), None, t)
        else:
            step.append(K[:, :, t:t + 1].contiguous(), V[:, :, t:t + 1].contiguous(), t)
    torch.cuda.synchronize()
    assert_bytes_equal(gpu_buffers(step), gpu_buffers(bulk), fmt)


def test_turbo_small_and_bulk_append_kernels_agree():
    """TurboQuant appends of at most 2048 rows take a latency-oriented kernel, larger
    ones a persistent one; both must write the same bytes (and the oracle's)."""
    cfg = SMALL["turbo"].scaled(context=1100)
    print("[turbo small vs bulk]", flush=True)
    bulk, K, V = _build(cfg, chunks=1)  # 2 x 2 x 1100 = 4400 rows in one append
    small = new_cache(cfg)
    for t0 in range(0, cfg.context, 100):  # 400 rows per append
        small.append(K[:, :, t0:t0 + 100].contiguous(), V[:, :, t0:t0 + 100].contiguous(), t0)
    torch.cuda.synchronize()
    got = gpu_buffers(small)
    assert_bytes_equal(got, gpu_buffers(bulk), "turbo small vs bulk")
    want = oracle_encode(cfg, host64(K), host64(V), oracle_constants(cfg))
    assert_bytes_equal(got, want, "turbo small vs oracle")


@pytest.mark.parametrize("fmt", ["kivi2", "fp4", "qjl1", "turbo", "latent"])
def test_split_count_invariance_and_determinism(fmt):
    cfg = SMALL[fmt]
    cache, _, _ = _build(cfg)
    q = synth.make_queries(cfg, device="cuda")
    lens = torch.from_numpy(synth.seq_lens_for(cfg)).cuda()
    outs = [cache.decode(q, lens, softmax_scale(cfg), splits=s).cpu().numpy() for s in (1, 0, 5, 0)]
    np.testing.assert_array_equal(outs[1], outs[3])
    # The matrix-core kernels (every format here) feed softmax weights to the PV
    # product in fp16, so each split configuration moves an output channel by up
    # to 2^-11 of the largest value it averages; two configurations differ by up
    # to twice that, 9.8e-4 (measured: 2.9e-4 to 5.6e-4).  A split-boundary bug
    # (a token lost or counted twice) shows as ~1e-1.
    tol = 1e-3
    errs = [float(row_rel_err(o, outs[0]).max()) for o in outs[:3]]
    print(f"  {fmt}: split configurations differ by {max(errs):.2e}", flush=True)
    assert max(errs) < tol


@pytest.mark.parametrize("fmt", ["fp4", "qjl1", "turbo"])
def test_fp32_inputs(fmt):
    """fp32 K/V (values not representable in bf16) go through the same formats."""
    cfg = SMALL[fmt].scaled(in_dtype="f32", context=200)
    cache, K, V = _build(cfg, chunks=1)
    want = oracle_encode(cfg, host64(K), host64(V), oracle_constants(cfg))
    assert_bytes_equal(gpu_buffers(cache), want, fmt + "/f32")


@pytest.mark.parametrize("fmt", ["fp4", "qjl1", "turbo"])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_mfma_group_sizes(fmt, G):
    """Every query-group size the matrix-core kernels are built for (TurboQuant with 16
    heads per KV head takes the general kernel), with a ragged tail."""
    cfg = SMALL[fmt].scaled(hq=2 * G, hkv=2, context=611)
    cache, K, V = _build(cfg, chunks=1)
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V), consts)
    q = synth.make_queries(cfg, device="cuda")
    lens = np.array([611, 97], dtype=np.int32)
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention(fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, consts)
    err = row_rel_err(out, ref)
    print(f"  {fmt} G={G} max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


def test_fp4_fp32_queries():
    """fp32 queries take the general kernel; same bar."""
    cfg = SMALL["fp4"].scaled(q_dtype="f32", context=300)
    cache, K, V = _build(cfg, chunks=1)
    enc = oracle_encode(cfg, host64(K), host64(V), {})
    q = synth.make_queries(cfg, device="cuda")
    lens = synth.seq_lens_for(cfg)
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention("fp4", enc, host64(q), lens, softmax_scale(cfg), cfg.hkv)
    assert row_rel_err(out, ref).max() <= RTOL


@pytest.mark.parametrize("hq", [32, 64])
def test_latent_head_counts(hq):
    """The latent matrix-core kernel at 1 and 2 waves per workgroup, ragged lengths."""
    cfg = SMALL["latent"].scaled(hq=hq, context=433)
    cache, K, _ = _build(cfg, chunks=1)
    enc = oracle_encode(cfg, host64(K), None, {})
    q = synth.make_queries(cfg, device="cuda")
    lens = np.array([433, 40], dtype=np.int32)
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention("latent", enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, {},
                              latent_dim=cfg.head_dim)
    err = row_rel_err(out, ref)
    print(f"  latent hq={hq} max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


@pytest.mark.parametrize("fmt", ["fp4", "qjl1", "latent", "kivi2", "turbo"])
def test_growing_logits_rescale(fmt):
    """Keys that grow along the context push every later tile's maximum logit past
    the running one, so the online-softmax rescale runs many times per split."""
    cfg = SMALL[fmt].scaled(context=640 if fmt == "kivi2" else 700)
    cache, K, V = _build(cfg, chunks=1, ramp=12.0)
    consts = oracle_constants(cfg)
    if fmt == "latent":
        enc = oracle_encode(cfg, host64(K), None, consts)
    else:
        enc = oracle_encode(cfg, host64(K), host64(V), consts)
    q = synth.make_queries(cfg, device="cuda")
    lens = synth.seq_lens_for(cfg, ragged=True)
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention(fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, consts,
                              latent_dim=cfg.head_dim)
    err = row_rel_err(out, ref)
    print(f"  {fmt} ramped keys: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


MULTI = [("fp4", 2), ("fp4", 3), ("fp4", 4), ("fp4", 5), ("fp4", 9), ("kivi2", 3), ("turbo", 2), ("qjl1", 5),
         ("qjl1", 2), ("qjl1", 3), ("turbo", 5), ("latent", 3),
         ("latent", 2)]


@pytest.mark.parametrize("fmt,nq", MULTI)
def test_multi_query_decode_matches_oracle(fmt, nq):
    """nq query tokens per sequence, query j over the first L - (nq - 1 - j)
    tokens: FP4 and QJL keys run on the matrix cores, 16 (query, head) pairs per
    launch (G = 4: nq = 3 fills 12 of 16 columns, nq = 5 takes 16 + 4, nq = 9 takes
    16 + 16 + 4; QJL columns repeat a pair per piece slot), the other formats on the
    general kernel.  Ragged lengths, one of them nq."""
    cfg = SMALL[fmt]
    print(f"[multi-query] {fmt} nq={nq} {cfg}", flush=True)
    cache, K, V = _build(cfg)
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), None if fmt == "latent" else host64(V), consts)
    q = synth.make_queries(cfg.scaled(hq=nq * cfg.hq), device="cuda")
    q = q.view(cfg.batch, nq, cfg.hq, q.shape[-1])
    lens = synth.seq_lens_for(cfg, ragged=True)
    lens[-1] = nq                                       # the first query sees one token
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention_multi(fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, consts,
                                    latent_dim=cfg.head_dim)
    err = row_rel_err(out.reshape(-1, out.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


WINDOWS = [("fp4", 16, 64, 1, 0), ("fp4", 0, 100, 3, 0), ("fp4", 40, 0, 1, 0), ("fp4", 300, 700, 2, 0),
           ("qjl1", 16, 64, 1, 0), ("qjl1", 24, 40, 3, 0),
           ("kivi2", 16, 64, 1, 0), ("kivi2", 8, 20, 2, 0), ("kivi2", 0, 5, 1, 0),
           ("turbo", 16, 64, 1, 0), ("turbo", 40, 100, 2, 0), ("turbo", 5, 0, 1, 0), ("turbo", 300, 700, 1, 0),
           ("turbo", 16, 64, 1, kvq.DECODE_FP32)]


@pytest.mark.parametrize("fmt,sink,recent,nq,flags", WINDOWS)
def test_mixed_precision_decode_matches_oracle(fmt, sink, recent, nq, flags):
    """bf16 sink and recent windows over a packed history.  Each sequence is
    appended to its own (ragged) length, its last tokens one at a time so that
    the recent ring wraps; one window covers whole sequences.  KIVI-2: the
    sequences end inside a key group, so staged keys outside a short recent
    window attend exact.  TurboQuant: the history's output goes back through
    R^T and the window's does not (matrix-core kernel, and the general one
    under DECODE_FP32)."""
    cfg = SMALL[fmt] if fmt != "kivi2" else SMALL[fmt].scaled(batch=3)
    print(f"[mixed] {fmt} sink={sink} recent={recent} nq={nq} flags={flags} {cfg}", flush=True)
    torch.manual_seed(0)
    consts = oracle_constants(cfg)
    cache = new_cache(cfg, sink_tokens=sink, recent_tokens=recent)
    K, V = inputs(cfg)
    lens = synth.seq_lens_for(cfg, ragged=True)
    lens[-1] = max(nq, 3)
    if fmt == "kivi2":
        lens[0] -= 7                                    # 25 keys of the last group staged
    for b in range(cfg.batch):
        seq, L = cache.sequence(b), int(lens[b])
        bulk = max(0, L - 5)
        if bulk:
            seq.append(K[b:b + 1, :, :bulk].contiguous(), V[b:b + 1, :, :bulk].contiguous(), 0)
        for t in range(bulk, L):
            seq.append(K[b:b + 1, :, t:t + 1].contiguous(), V[b:b + 1, :, t:t + 1].contiguous(), t)
    torch.cuda.synchronize()
    enc = oracle_encode(cfg, host64(K), host64(V), consts)
    q = synth.make_queries(cfg.scaled(hq=nq * cfg.hq), device="cuda").view(cfg.batch, nq, cfg.hq, -1)
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg), flags=flags).cpu().numpy()
    ref = OA.decode_attention_mixed(fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, host64(K), host64(V),
                                    sink, recent, consts)
    err = row_rel_err(out.reshape(-1, out.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


RAGGED = [("fp4", {}), ("kivi2", {}), ("turbo", {}), ("qjl1", {}), ("latent", {}),
          ("fp4", {"sink_tokens": 8, "recent_tokens": 16}), ("qjl1", {"sink_tokens": 40, "recent_tokens": 4})]


@pytest.mark.parametrize("fmt,win", RAGGED)
def test_ragged_append_equals_per_sequence_appends(fmt, win):
    """One append with a first position per sequence writes exactly the bytes
    that one append per sequence at that position writes (bf16 windows too)."""
    cfg = SMALL[fmt].scaled(batch=2)
    print(f"[ragged append] {fmt} {win} {cfg}", flush=True)
    K, V = inputs(cfg)
    n = 32 if fmt == "kivi2" else 20
    starts = [0, 64] if fmt == "kivi2" else [37, 3]
    a, b = new_cache(cfg, **win), new_cache(cfg, **win)
    if fmt == "latent":
        a.append(K[:, :n].contiguous(), None, starts)
        for s in range(cfg.batch):
            b.sequence(s).append(K[s:s + 1, :n].contiguous(), None, starts[s])
    else:
        a.append(K[:, :, :n].contiguous(), V[:, :, :n].contiguous(), starts)
        for s in range(cfg.batch):
            b.sequence(s).append(K[s:s + 1, :, :n].contiguous(), V[s:s + 1, :, :n].contiguous(), starts[s])
    torch.cuda.synchronize()
    for name in a.bufs:
        assert torch.equal(a.bufs[name], b.bufs[name]), name


def test_ragged_append_beyond_one_launch():
    """300 sequences: the positions go to the kernels by value, 256 sequences per
    launch; every sequence's bytes match its own append."""
    cfg = C["fp4_b16_t32k"].scaled(batch=300, hq=1, hkv=1, context=64)
    print(f"[ragged append 300] {cfg}", flush=True)
    K, V = synth.make_kv(cfg, 0, 300, 0, 3, device="cuda")
    rng = np.random.default_rng(3)
    starts = rng.integers(0, 62, 300).tolist()
    a, b = new_cache(cfg), new_cache(cfg)
    a.append(K.contiguous(), V.contiguous(), starts)
    for s in range(300):
        b.sequence(s).append(K[s:s + 1].contiguous(), V[s:s + 1].contiguous(), starts[s])
    torch.cuda.synchronize()
    for name in a.bufs:
        assert torch.equal(a.bufs[name], b.bufs[name]), name


@pytest.mark.parametrize("nq", [1, 2])
def test_kivi_unaligned_appends_and_staged_decode(nq):
    """KIVI-2 appended in uneven chunks down to single tokens: every whole key
    group and every value is coded exactly as the oracle codes them, and decode
    reads each sequence's incomplete last group from the staged keys."""
    cfg = SMALL["kivi2"].scaled(batch=3)
    print(f"[kivi staging] nq={nq} {cfg}", flush=True)
    cache = new_cache(cfg)
    K, V = inputs(cfg)
    lens = np.array([256, 75, 9], dtype=np.int32)
    chunks = [5, 27, 40, 1, 1, 3, 31, 64]
    for b in range(cfg.batch):
        seq, t = cache.sequence(b), 0
        for ci in range(100):
            if t >= lens[b]:
                break
            n = min(chunks[ci % len(chunks)], int(lens[b]) - t)
            seq.append(K[b:b + 1, :, t:t + n].contiguous(), V[b:b + 1, :, t:t + n].contiguous(), t)
            t += n
    torch.cuda.synchronize()
    want = oracle_encode(cfg, host64(K), host64(V), {})
    got = gpu_buffers(cache)
    for b in range(cfg.batch):
        L, Lg = int(lens[b]), int(lens[b]) // 32 * 32
        np.testing.assert_array_equal(got["k_codes"][b, :, :Lg], want["k_codes"][b, :, :Lg])
        np.testing.assert_array_equal(got["k_scale"][b, :, :Lg // 32], want["k_scale"][b, :, :Lg // 32])
        np.testing.assert_array_equal(got["k_zero"][b, :, :Lg // 32], want["k_zero"][b, :, :Lg // 32])
        for name in ("v_codes", "v_scale", "v_zero"):
            np.testing.assert_array_equal(got[name][b, :, :L], want[name][b, :, :L])
    q = synth.make_queries(cfg.scaled(hq=nq * cfg.hq), device="cuda").view(cfg.batch, nq, cfg.hq, -1)
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention_kivi_staged(want, host64(q), lens, softmax_scale(cfg), cfg.hkv, host64(K))
    err = row_rel_err(out.reshape(-1, out.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL
    # shorter prefixes of the same sequences: groups the appends completed are read coded
    short = np.maximum(lens - np.array([100, 20, 6], dtype=np.int32), nq).astype(np.int32)
    out = cache.decode(q, torch.from_numpy(short).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention_kivi_staged(want, host64(q), short, softmax_scale(cfg), cfg.hkv, host64(K), lens)
    err = row_rel_err(out.reshape(-1, out.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    print(f"  prefixes: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


def test_kivi_ragged_unaligned_append_equals_per_sequence():
    """A ragged KIVI-2 append with starts inside key groups writes the bytes
    (codes, staged keys) of one append per sequence."""
    cfg = SMALL["kivi2"].scaled(batch=2)
    K, V = inputs(cfg)
    a, b = new_cache(cfg), new_cache(cfg)
    for c in (a, b):  # earlier tokens of each sequence: 37 and 70 of them
        c.sequence(0).append(K[0:1, :, :37].contiguous(), V[0:1, :, :37].contiguous(), 0)
        c.sequence(1).append(K[1:2, :, :70].contiguous(), V[1:2, :, :70].contiguous(), 0)
    a.append(K[:, :, 100:120].contiguous(), V[:, :, 100:120].contiguous(), [37, 70])
    b.sequence(0).append(K[0:1, :, 100:120].contiguous(), V[0:1, :, 100:120].contiguous(), 37)
    b.sequence(1).append(K[1:2, :, 100:120].contiguous(), V[1:2, :, 100:120].contiguous(), 70)
    torch.cuda.synchronize()
    for name in a.bufs:
        assert torch.equal(a.bufs[name], b.bufs[name]), name


@pytest.mark.parametrize("fmt", ["turbo", "qjl1"])
def test_wide_range_queries(fmt):
    """Queries whose channels span 2^-12 .. 2^3 (and some exact zeros): every
    32-element block of the bit-key products' query operand then needs all its
    pieces, each at its own power-of-two scale."""
    cfg = SMALL[fmt]
    cache, K, V = _build(cfg)
    consts = oracle_constants(cfg)
    enc = oracle_encode(cfg, host64(K), host64(V), consts)
    g = torch.Generator().manual_seed(7)
    q0 = synth.make_queries(cfg, device="cpu")
    mult = torch.exp2(torch.empty(q0.shape).uniform_(-12.0, 3.0, generator=g))
    mult[..., ::11] = 0.0
    q = (q0.float() * mult).to(q0.dtype).cuda()
    lens = synth.seq_lens_for(cfg, ragged=True)
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention(fmt, enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, consts,
                              latent_dim=cfg.head_dim)
    err = row_rel_err(out, ref)
    print(f"  {fmt} wide-range queries: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL


@pytest.mark.parametrize("fmt", ["fp4", "qjl1", "turbo", "latent", "kivi2"])
def test_graph_replay_matches_eager(fmt):
    """Append + decode captured as a HIP graph: every replay, with eager work and
    synchronisations in between, reproduces the eager result bit for bit."""
    cfg = SMALL[fmt]
    cache, K, V = _build(cfg)
    q = synth.make_queries(cfg, device="cuda")
    lens = torch.from_numpy(synth.seq_lens_for(cfg)).cuda()
    n = 32 if fmt == "kivi2" else 1
    t0 = cfg.context - n
    if fmt == "latent":
        kn, vn = K[:, t0:].contiguous(), None
    else:
        kn, vn = K[:, :, t0:].contiguous(), V[:, :, t0:].contiguous()
    out = torch.empty(cfg.batch, cfg.hq, cfg.head_dim, dtype=torch.float32, device="cuda")
    ws = torch.zeros(cache.workspace_bytes(cfg.hq, cfg.context, 0, q.dtype), dtype=torch.uint8, device="cuda")

    def step():
        cache.append(kn, vn, t0)
        cache.decode(q, lens, softmax_scale(cfg), out=out, ws=ws)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


@pytest.mark.parametrize("fmt", ["fp4", "qjl1", "turbo", "latent"])
def test_repeated_decode_bit_identical(fmt):
    """Many tiles per wave on both halves of each LDS ring: repeated decodes of the
    same cache must agree bit for bit (a read of a ring stage before its loads
    land shows up here as run-to-run differences)."""
    cfg = SMALL[fmt].scaled(batch=4, context=12288)
    cache, _, _ = _build(cfg, chunks=3)
    q = synth.make_queries(cfg, device="cuda")
    lens = torch.full((cfg.batch,), cfg.context, dtype=torch.int32, device="cuda")
    ref = cache.decode(q, lens, softmax_scale(cfg), splits=4)
    torch.cuda.synchronize()
    for _ in range(12):
        out = cache.decode(q, lens, softmax_scale(cfg), splits=4)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
