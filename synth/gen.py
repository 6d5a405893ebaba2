"""Seeded generators for K/V/latent/query tensors and the methods' Gaussian draws.

Values are standard normal draws (torch's generator on the requested device),
with a fixed set of outlier key channels per KV head multiplied in fp32 before
the cast to the input dtype (a keys-only outlier pattern, as the KIVI paragraph
of the "TurboQuant vs OSCAR vs EpiCache" page describes).  Token ranges are
drawn in blocks of BLOCK tokens with a seed of their own, so any sub-range of a
large cache can be regenerated without drawing the rest.

A CPU generator and a GPU generator give different streams for the same seed:
a test that needs the same values on both sides draws once and copies.
"""

import numpy as np
import torch

BLOCK = 4096
_MASK = (1 << 63) - 1

# stream ids
_S_K, _S_V, _S_Q, _S_OUT, _S_LAT, _S_IDX = 1, 2, 3, 4, 5, 6


def _mix(*vals: int) -> int:
    """splitmix64 over a tuple of ints -> 63-bit seed."""
    h = 0x9E3779B97F4A7C15
    for v in vals:
        z = (h ^ (int(v) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        z = (z + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        h = z ^ (z >> 31)
    return h & _MASK


def _gen(device, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*key))
    return g


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def outlier_channels(cfg) -> torch.Tensor:
    """int64 [hkv, n_outlier]: the fixed outlier key channels of each KV head."""
    out = torch.zeros(cfg.hkv, cfg.n_outlier, dtype=torch.int64)
    for h in range(cfg.hkv):
        g = _gen("cpu", cfg.seed, _S_OUT, h)
        out[h] = torch.randperm(cfg.head_dim, generator=g)[: cfg.n_outlier].sort().values
    return out


def _normal_tokens(cfg, stream, b, h, t0, t1, width, device) -> torch.Tensor:
    """fp32 [t1-t0, width] standard normals for (stream, b, h), blockwise seeded."""
    rows = []
    blk0, blk1 = t0 // BLOCK, (t1 + BLOCK - 1) // BLOCK
    for blk in range(blk0, blk1):
        g = _gen(device, cfg.seed, stream, b, h, blk)
        x = torch.randn(BLOCK, width, generator=g, device=device, dtype=torch.float32)
        lo = max(t0, blk * BLOCK) - blk * BLOCK
        hi = min(t1, (blk + 1) * BLOCK) - blk * BLOCK
        rows.append(x[lo:hi])
    if not rows:
        return torch.empty(0, width, device=device, dtype=torch.float32)
    return torch.cat(rows, 0)


def make_kv(cfg, b0=0, b1=None, t0=0, t1=None, device="cpu"):
    """K, V of shape [b1-b0, hkv, t1-t0, head_dim] in the config's input dtype."""
    b1 = cfg.batch if b1 is None else b1
    t1 = cfg.context if t1 is None else t1
    dt = _torch_dtype(cfg.in_dtype)
    nb, nt = b1 - b0, t1 - t0
    K = torch.empty(nb, cfg.hkv, nt, cfg.head_dim, dtype=dt, device=device)
    V = torch.empty_like(K)
    outl = outlier_channels(cfg).to(device)
    for i, b in enumerate(range(b0, b1)):
        for h in range(cfg.hkv):
            k = _normal_tokens(cfg, _S_K, b, h, t0, t1, cfg.head_dim, device)
            if cfg.n_outlier:
                k[:, outl[h]] *= cfg.outlier_scale
            K[i, h] = k.to(dt)
            V[i, h] = _normal_tokens(cfg, _S_V, b, h, t0, t1, cfg.head_dim, device).to(dt)
    return K, V


def make_latent(cfg, b0=0, b1=None, t0=0, t1=None, device="cpu"):
    """[b1-b0, t1-t0, head_dim + rope_dim] bf16: the latent, then the RoPE key."""
    b1 = cfg.batch if b1 is None else b1
    t1 = cfg.context if t1 is None else t1
    out = torch.empty(b1 - b0, t1 - t0, cfg.key_width, dtype=torch.bfloat16, device=device)
    for i, b in enumerate(range(b0, b1)):
        out[i] = _normal_tokens(cfg, _S_LAT, b, 0, t0, t1, cfg.key_width, device).to(torch.bfloat16)
    return out


def make_queries(cfg, device="cpu"):
    """[batch, hq, key_width] in the config's query dtype."""
    g = _gen(device, cfg.seed, _S_Q)
    q = torch.randn(cfg.batch, cfg.hq, cfg.key_width, generator=g, device=device, dtype=torch.float32)
    return q.to(_torch_dtype(cfg.q_dtype))


def gaussian_matrix(seed: int, rows: int, cols: int, stream: int = 0) -> np.ndarray:
    """float64 [rows, cols] iid N(0,1) (NumPy PCG64), for the methods' own random draws."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77, stream])))
    return rng.standard_normal((rows, cols))


def seq_lens_for(cfg, ragged: bool = False, seed: int = 0) -> np.ndarray:
    """int32 [batch] context lengths: all equal to cfg.context, or a seeded ragged mix."""
    if not ragged:
        return np.full(cfg.batch, cfg.context, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 91, seed])))
    lens = rng.integers(1, cfg.context + 1, size=cfg.batch).astype(np.int32)
    lens[0] = cfg.context
    return lens


def make_indexer_scores(seed: int, batch: int, length: int, layer: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [batch, length] stand-ins for a sparse indexer's scores: N(0, 1)
    background with a few raised spans per sequence (the positions a query would
    look back at), rounded to bf16 values as a low-precision indexer emits them,
    so that equal scores occur.  `layer` draws an independent set."""
    out = torch.empty(batch, length, dtype=torch.float32, device=device)
    for b in range(batch):
        g = _gen(device, seed, _S_IDX, layer, b)
        x = torch.randn(length, generator=g, device=device, dtype=torch.float32)
        nspan = 8
        starts = torch.randint(0, max(1, length), (nspan,), generator=g, device=device)
        lens = torch.randint(16, 512, (nspan,), generator=g, device=device)
        lift = 2.0 + 2.0 * torch.rand(nspan, generator=g, device=device)
        for i in range(nspan):
            s0 = int(starts[i])
            x[s0:s0 + int(lens[i])] += float(lift[i])
        out[b] = x.to(torch.bfloat16).to(torch.float32)
    return out
