"""kv_decode_attention_static (the decode entry point that allocates nothing)
against kv_decode_attention on the same caches and queries, through the C ABI:
the two share every kernel and the split plan, so outputs must be identical.
Two calls in a row on one GPU, the second with a smaller input, check that the
shared scratch array carries nothing from one call into the next."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from bit_kv_cache_04_amd import kvq
from gpu_helpers import inputs, new_cache, softmax_scale

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


def _static(cache, q, lens, scale, out, nq=1):
    opts = kvq.KVDecodeOpts(0, None, None, nq, 0)
    st = kvq.lib().kv_decode_attention_static(
        ctypes.byref(cache.struct), ctypes.c_void_p(q.data_ptr()), kvq.DT_BF16 if q.dtype == torch.bfloat16
        else kvq.DT_F32, q.shape[-2], ctypes.c_void_p(lens.data_ptr()), cache.T,
        ctypes.c_float(scale), ctypes.c_void_p(out.data_ptr()), ctypes.byref(opts),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, kvq.STATUS.get(st, st)
    return out


def _case(cfg, seed):
    cache = new_cache(cfg)
    K, V = inputs(cfg)
    if cfg.fmt == "latent":
        cache.append(K, None, 0)
    else:
        cache.append(K, V, 0)
    q = synth.make_queries(cfg.scaled(seed=cfg.seed + seed), device="cuda")
    lens = torch.from_numpy(synth.seq_lens_for(cfg, ragged=True, seed=seed)).cuda()
    return cache, q, lens


@pytest.mark.parametrize("fmt,big,small", [
    ("fp4", dict(batch=4, hq=16, hkv=4, context=2000), dict(batch=2, hq=8, hkv=2, context=300)),
    ("turbo", dict(batch=3, hq=16, hkv=2, context=1500), dict(batch=1, hq=8, hkv=1, context=100)),
    ("latent", dict(batch=3, hq=128, context=700), dict(batch=1, hq=64, context=90)),
    ("kivi2", dict(batch=2, hq=8, hkv=2, context=512), dict(batch=1, hq=4, hkv=2, context=64)),
])
def test_static_workspace_decode_equals_workspace_decode(fmt, big, small):
    base = {"fp4": C["fp4_b16_t32k"], "turbo": C["turbo_b8_t128k"], "latent": C["latent_b64_t64k"],
            "kivi2": C["kivi2_tiny"]}[fmt]
    for i, shape in enumerate((big, small)):
        cfg = base.scaled(**shape)
        print(f"[static decode] {fmt} call {i} {shape}", flush=True)
        cache, q, lens = _case(cfg, i)
        scale = softmax_scale(cfg)
        want = cache.decode(q, lens, scale)
        got = torch.full_like(want, float("nan"))
        _static(cache, q, lens, scale, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{fmt} call {i}: {(got - want).abs().max().item()}"


def test_static_workspace_several_queries():
    cfg = C["fp4_b16_t32k"].scaled(batch=2, hq=8, hkv=2, context=400)
    cache, _, lens = _case(cfg, 0)
    q = synth.make_queries(cfg.scaled(hq=3 * cfg.hq), device="cuda").view(cfg.batch, 3, cfg.hq, -1)
    want = cache.decode(q, lens, softmax_scale(cfg))
    got = torch.full_like(want, float("nan"))
    _static(cache, q, lens, softmax_scale(cfg), got, nq=3)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
