"""KIVI-2 decode at 64 and 128 channels on the matrix cores against the oracle.

The matrix-core kernel reads the coded key groups of each sequence; the
tokens of its incomplete last group (keys still in staging) take one more
split in fp32 (a last grid column of the same launch on small grids, the
general kernel on large ones).  Every case appends in uneven chunks, so the
sequences end inside a key group, and compares with the oracle's staged
reference (page "TurboQuant vs OSCAR vs EpiCache", section "quantization
frontiers", KIVI paragraph: keys per channel, values per token, 2 bits).
"""

import numpy as np
import pytest
import torch

import synth
from bit_kv_cache_04_amd import kvq
from gpu_helpers import (RTOL, gpu_buffers, host64, inputs, new_cache, oracle_encode, row_rel_err,
                         softmax_scale)
from oracle import attention as OA

pytestmark = pytest.mark.gpu

BASE = synth.CONFIGS["kivi2_tiny"].scaled(head_dim=128, hkv=2, hq=8, context=1024, batch=3)
CHUNKS = [5, 27, 40, 1, 3, 31, 64, 200]


def _appended(cfg, lens, ramp=None):
    """A cache holding lens[b] tokens of each sequence, appended in uneven chunks."""
    torch.manual_seed(0)
    cache = new_cache(cfg)
    K, V = inputs(cfg)
    if ramp is not None:
        r = 1.0 + ramp * torch.arange(cfg.context, device=K.device, dtype=torch.float32) / cfg.context
        K = (K.float() * r.view(1, 1, -1, 1)).to(K.dtype)
    for b in range(cfg.batch):
        seq, t, ci = cache.sequence(b), 0, b
        while t < lens[b]:
            n = min(CHUNKS[ci % len(CHUNKS)], int(lens[b]) - t)
            seq.append(K[b:b + 1, :, t:t + n].contiguous(), V[b:b + 1, :, t:t + n].contiguous(), t)
            t += n
            ci += 1
    torch.cuda.synchronize()
    return cache, K, V


def _check(cfg, lens, nq=1, splits=0, flags=0, ramp=None, decode_lens=None, what=""):
    cache, K, V = _appended(cfg, lens, ramp)
    want = oracle_encode(cfg, host64(K), host64(V), {})
    q = synth.make_queries(cfg.scaled(hq=nq * cfg.hq), device="cuda").view(cfg.batch, nq, cfg.hq, -1)
    dl = lens if decode_lens is None else decode_lens
    out = cache.decode(q, torch.from_numpy(dl).cuda(), softmax_scale(cfg), splits=splits, flags=flags)
    out = out.cpu().numpy().reshape(cfg.batch, nq, cfg.hq, -1)
    ref = OA.decode_attention_kivi_staged(want, host64(q), dl, softmax_scale(cfg), cfg.hkv, host64(K), lens)
    err = row_rel_err(out.reshape(-1, out.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    print(f"  {what} max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G,nq", [(1, 1), (2, 1), (4, 1), (8, 2), (16, 1), (32, 1), (4, 5)])
def test_kivi_matrix_cores_match_oracle(G, nq, d):
    """Head groups of 1 to 32 and several queries per sequence (more than 16
    (query, head) pairs take several launches), ragged lengths ending inside a
    key group, with outlier key channels, at 64 and 128 channels."""
    cfg = BASE.scaled(hq=G * BASE.hkv, head_dim=d)
    lens = np.array([1024, 517, 33], dtype=np.int32)
    print(f"[kivi mfma] d={d} G={G} nq={nq} lens={lens.tolist()}", flush=True)
    _check(cfg, lens, nq=nq, what=f"d={d} G={G} nq={nq}")


@pytest.mark.parametrize("d", [64, 128])
def test_kivi_short_sequences_and_split_counts(d):
    """Sequences shorter than one key group (staged tokens only), exactly one
    group, and one token; the result does not depend on the split count."""
    cfg = BASE.scaled(hq=4 * BASE.hkv, batch=4, head_dim=d)
    lens = np.array([1, 31, 32, 800], dtype=np.int32)
    print(f"[kivi short] d={d} lens={lens.tolist()}", flush=True)
    outs = [_check(cfg, lens, splits=s, what=f"splits={s}") for s in (0, 1, 5)]
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=0, atol=1e-3 * np.abs(outs[0]).max())


@pytest.mark.parametrize("d", [64, 128])
def test_kivi_matrix_cores_agree_with_the_fp32_kernel(d):
    """The same cache on the fp32 general kernel (every split reads through it)."""
    cfg = BASE.scaled(hq=4 * BASE.hkv, head_dim=d)
    lens = np.array([1000, 259, 70], dtype=np.int32)
    print(f"[kivi fp32] d={d} lens={lens.tolist()}", flush=True)
    a = _check(cfg, lens, what="matrix cores")
    b = _check(cfg, lens, flags=kvq.DECODE_FP32, what="fp32 kernel")
    np.testing.assert_allclose(a, b, rtol=0, atol=2e-3 * np.abs(b).max())


@pytest.mark.parametrize("d", [64, 128])
def test_kivi_growing_logits_rescale(d):
    """Keys growing along the sequence move the running max often."""
    cfg = BASE.scaled(hq=4 * BASE.hkv, batch=2, head_dim=d)
    lens = np.array([1024, 700], dtype=np.int32)
    print(f"[kivi ramp] d={d}", flush=True)
    _check(cfg, lens, ramp=12.0, what="ramped keys")


def test_kivi_prefixes_of_appended_sequences():
    """Decoding shorter prefixes than were appended: the groups the appends
    completed are read coded, up to each prefix's end."""
    cfg = BASE.scaled(hq=4 * BASE.hkv)
    lens = np.array([1024, 517, 90], dtype=np.int32)
    short = np.array([1000, 300, 64], dtype=np.int32)
    print(f"[kivi prefixes] {short.tolist()} of {lens.tolist()}", flush=True)
    _check(cfg, lens, decode_lens=short, what="prefixes")


def test_kivi_bytes_still_match_after_decode():
    """Decode reads the cache only: the coded bytes stay the oracle's."""
    cfg = BASE.scaled(hq=4 * BASE.hkv, batch=2)
    lens = np.array([1024, 99], dtype=np.int32)
    cache, K, V = _appended(cfg, lens)
    want = oracle_encode(cfg, host64(K), host64(V), {})
    q = synth.make_queries(cfg, device="cuda")
    cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg))
    got = gpu_buffers(cache)
    for b in range(cfg.batch):
        L, Lg = int(lens[b]), int(lens[b]) // 32 * 32  # keys of the incomplete group wait in staging
        np.testing.assert_array_equal(got["k_codes"][b, :, :Lg], want["k_codes"][b, :, :Lg])
        np.testing.assert_array_equal(got["k_scale"][b, :, :Lg // 32], want["k_scale"][b, :, :Lg // 32])
        np.testing.assert_array_equal(got["v_codes"][b, :, :L], want["v_codes"][b, :, :L])


@pytest.mark.parametrize("d", [64, 128])
def test_kivi_large_grid_staged_tail_on_the_general_kernel(d):
    """A grid of at least 256 workgroups leaves the staged tokens to the general
    kernel (small grids take them in a last column of the same launch) and reads
    the prepared query copy: 16 sequences x 8 KV heads, lengths ending inside a
    key group."""
    cfg = BASE.scaled(batch=16, hkv=8, hq=32, context=4096, head_dim=d)
    lens = np.array([4096 - 5 * b - (b % 3) * 11 for b in range(16)], dtype=np.int32)
    print(f"[kivi large grid] d={d} lens={lens.tolist()}", flush=True)
    _check(cfg, lens, what="large grid")


@pytest.mark.parametrize("d", [64, 128])
def test_kivi_bf16_queries(d):
    """bf16 queries on a small grid (the prepared fp32 copy, not the caller's
    queries, feeds the kernel), with several queries per sequence."""
    cfg = BASE.scaled(hq=4 * BASE.hkv, head_dim=d, q_dtype="bf16")
    lens = np.array([1000, 300, 45], dtype=np.int32)
    print(f"[kivi bf16 q] d={d} lens={lens.tolist()}", flush=True)
    _check(cfg, lens, nq=2, what="bf16 queries")
