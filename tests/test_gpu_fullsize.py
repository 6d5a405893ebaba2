"""GPU parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (default split plan, every sequence and head in one call).

The cache is filled the way bench.py fills it (untimed prefill in 16K-token
chunks per sequence, then the step's own append of the last tokens).  The oracle
then re-encodes sampled (sequence, KV head) units from the same seeded inputs and
decodes their query heads:
  - every packed byte of a sampled unit must equal the oracle's;
  - every output row of a sampled unit must be within 2e-3 max relative error.
Inputs are drawn on the GPU and copied to the host, so both sides see the same
values.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import RTOL, assert_bytes_equal, library_constants, oracle_constants, oracle_encode, row_rel_err, \
    softmax_scale
from bit_kv_cache_04_amd.cache import PackedKVCache
from oracle import attention as OA

pytestmark = pytest.mark.gpu

CHUNK = 16384


def _n_new(cfg):
    return 32 if cfg.fmt == "kivi2" else max(1, cfg.append_new)


def _build_full(cfg):
    cache = PackedKVCache(cfg.fmt, cfg.batch, cfg.hkv, cfg.head_dim, cfg.context, cfg.rope_dim, device="cuda",
                          constants=library_constants(cfg))
    T, n_new = cfg.context, _n_new(cfg)
    n_pre = T - n_new
    for b in range(cfg.batch):
        seq = cache.sequence(b)
        for t0 in range(0, n_pre, CHUNK):
            t1 = min(n_pre, t0 + CHUNK)
            if cfg.fmt == "latent":
                seq.append(synth.make_latent(cfg, b, b + 1, t0, t1, device="cuda"), None, t0)
            else:
                K, V = synth.make_kv(cfg, b, b + 1, t0, t1, device="cuda")
                seq.append(K, V, t0)
    if cfg.fmt == "latent":
        cache.append(synth.make_latent(cfg, 0, cfg.batch, n_pre, T, device="cuda"), None, n_pre)
    else:
        K, V = synth.make_kv(cfg, 0, cfg.batch, n_pre, T, device="cuda")
        cache.append(K, V, n_pre)
    torch.cuda.synchronize()
    return cache


def _unit_inputs(cfg, b, h):
    """Host fp64 inputs of sequence b, KV head h over the whole context."""
    ks, vs = [], []
    for t0 in range(0, cfg.context, CHUNK):
        t1 = min(cfg.context, t0 + CHUNK)
        if cfg.fmt == "latent":
            ks.append(synth.make_latent(cfg, b, b + 1, t0, t1, device="cuda").double().cpu().numpy())
        else:
            K, V = synth.make_kv(cfg, b, b + 1, t0, t1, device="cuda")
            ks.append(K[:, h:h + 1].double().cpu().numpy())
            vs.append(V[:, h:h + 1].double().cpu().numpy())
    axis = 1 if cfg.fmt == "latent" else 2
    K = np.concatenate(ks, axis=axis)
    V = np.concatenate(vs, axis=axis) if vs else None
    return K, V


def _unit_bytes(cache, b, h):
    out = {}
    for name in cache.bufs:
        v = cache.view(name)
        out[name] = (v[b:b + 1] if cache.fmt == "latent" else v[b:b + 1, h:h + 1]).cpu().numpy()
    return out


WORKLOADS = ["kivi2_tiny", "fp4_b16_t32k", "turbo_b8_t128k", "qjl1_b1_t1m", "latent_b64_t64k"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_full_size_sampled_units(name):
    cfg = synth.CONFIGS[name]
    print(f"[full size] {name}", flush=True)
    cache = _build_full(cfg)
    q = synth.make_queries(cfg, device="cuda")
    lens = torch.full((cfg.batch,), cfg.context, dtype=torch.int32, device="cuda")
    out = cache.decode(q, lens, softmax_scale(cfg)).cpu().numpy()
    qh = q.double().cpu().numpy()
    consts = oracle_constants(cfg)
    G = cfg.group
    units = [(0, 0), (cfg.batch - 1, cfg.hkv - 1)]
    if cfg.fmt == "latent":
        units = [(0, 0), (cfg.batch - 1, 0)]
    if cfg.context > 200000:  # the oracle takes ~30 s per million-token unit
        units = [(cfg.batch - 1, cfg.hkv - 1)]
    for b, h in sorted(set(units)):
        unit = cfg.scaled(batch=1, hkv=1, hq=G)
        K, V = _unit_inputs(cfg, b, h)
        enc = oracle_encode(unit, K, V, consts)
        assert_bytes_equal(_unit_bytes(cache, b, h), enc, f"{name} unit ({b}, {h})")
        rows = slice(h * G, (h + 1) * G)
        ref = OA.decode_attention(cfg.fmt, enc, qh[b:b + 1, rows], [cfg.context], softmax_scale(cfg), 1, consts,
                                  latent_dim=cfg.head_dim)
        err = row_rel_err(out[b:b + 1, rows], ref)
        print(f"  unit ({b}, {h}): bytes equal, max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= RTOL
