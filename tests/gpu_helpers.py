"""Shared pieces of the GPU parity tests: build a cache through the C ABI, encode
the same inputs with the oracle, and compare.

Inputs come from `synth` (drawn on the GPU, copied to the host for the
oracle); the oracle's constants are its own (QR, Lloyd-Max, bf16 rounding),
the library's are made by libkvq's host helpers from the same Gaussian draws.
"""

import math

import numpy as np
import torch

import synth
from bit_kv_cache_04_amd.cache import PackedKVCache, make_constants
from oracle import attention as OA
from oracle import formats as OF
from oracle.lloyd_max import canonical_codebook
from oracle.rotation import canonical_projection, canonical_rotation

RTOL = 2e-3  # max relative error per output row, |o - o*|_max / |o*|_max


def gauss_pair(cfg):
    return (synth.gaussian_matrix(cfg.seed, cfg.head_dim, cfg.head_dim, stream=1),
            synth.gaussian_matrix(cfg.seed, 128, cfg.head_dim, stream=2))


def oracle_constants(cfg):
    g_rot, g_proj = gauss_pair(cfg)
    c = {}
    if cfg.fmt == "turbo":
        c["rot"] = canonical_rotation(g_rot)
        c["levels"], c["thresholds"] = canonical_codebook(2, cfg.head_dim)
    if cfg.fmt in ("turbo", "qjl1"):
        c["proj"] = canonical_projection(g_proj)
    return c


def library_constants(cfg):
    g_rot, g_proj = gauss_pair(cfg)
    return make_constants(cfg.fmt, cfg.head_dim, g_rot, g_proj)


def new_cache(cfg, capacity=None, **kw):
    return PackedKVCache(cfg.fmt, cfg.batch, cfg.hkv, cfg.head_dim, capacity or cfg.context, cfg.rope_dim,
                         device="cuda", constants=library_constants(cfg), **kw)


def inputs(cfg, device="cuda"):
    if cfg.fmt == "latent":
        return synth.make_latent(cfg, device=device), None
    return synth.make_kv(cfg, device=device)


def host64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64) if t is not None else None


def oracle_encode(cfg, K, V, consts, chunk=16384):
    """Oracle buffers for host fp64 inputs, encoded in token chunks to bound memory."""
    T = K.shape[-2]
    parts = []
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        if cfg.fmt == "latent":
            parts.append(OF.encode_cache("latent", latent=K[:, t0:t1], consts=consts, latent_dim=cfg.head_dim))
        else:
            parts.append(OF.encode_cache(cfg.fmt, K[:, :, t0:t1], V[:, :, t0:t1], consts=consts))
    out = {}
    for name in parts[0]:
        if cfg.fmt == "kivi2" and name in ("k_scale", "k_zero"):
            axis = 2
        else:
            axis = 1 if cfg.fmt == "latent" else 2
        out[name] = np.concatenate([p[name] for p in parts], axis=axis)
    return out


def gpu_buffers(cache, t0=0, t1=None):
    """Host copies of the cache's buffers (token range [t0, t1))."""
    t1 = cache.T if t1 is None else t1
    out = {}
    for name in cache.bufs:
        if name.startswith(("sink_", "recent_")) or name == "k_stage":
            continue  # bf16 windows: not packed token slots
        v = cache.view(name)
        if cache.fmt == "kivi2" and name in ("k_scale", "k_zero"):
            v = v[:, :, t0 // 32:t1 // 32]
        elif cache.fmt == "latent":
            v = v[:, t0:t1]
        else:
            v = v[:, :, t0:t1]
        out[name] = v.cpu().numpy()
    return out


def assert_bytes_equal(got, want, what=""):
    for name, w in want.items():
        g = got[name]
        assert g.shape == w.shape, (name, g.shape, w.shape)
        if g.dtype == np.float32:
            g = g.view(np.uint32)
            w = np.asarray(w, np.float32).view(np.uint32)
        else:
            w = np.asarray(w).astype(g.dtype)
        bad = np.count_nonzero(g != w)
        assert bad == 0, f"{what} {name}: {bad} of {g.size} elements differ"


def row_rel_err(got, want):
    """Per (b, hq) row: max |got - want| / max |want|."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = np.abs(got - want).max(-1)
    den = np.abs(want).max(-1)
    return num / np.maximum(den, 1e-30)


def softmax_scale(cfg):
    return 1.0 / math.sqrt(cfg.key_width)
