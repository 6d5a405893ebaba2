"""GPU parity of TurboQuant caches built on the structured rotation (Hadamard
transform with and without the bit-reversal permutation) instead of a Haar draw:
the append and decode kernels take any bf16-valued d x d matrix, so the packed
bytes must still equal the oracle's bit for bit and the outputs stay within the
2e-3 row bar, with and without loud key channels, on the matrix-core kernel
(8 query heads per KV head) and the general one (16).  The same with the
rotation applied as a Hadamard butterfly (layout.rotation, no matrix passed):
the append's fp64 sums of bf16 inputs are exact, so its bytes equal those of
the dense product; its first append (2,400 rows) takes the bulk append kernel,
the second (708 rows) the small one."""

import numpy as np
import pytest
import torch

import synth
from bit_kv_cache_04_amd import kvq
from bit_kv_cache_04_amd.cache import PackedKVCache, make_constants
from gpu_helpers import RTOL, assert_bytes_equal, gpu_buffers, host64, oracle_encode, row_rel_err, softmax_scale
from oracle import attention as OA
from oracle.lloyd_max import canonical_codebook
from oracle.rotation import canonical_hadamard_rotation, canonical_projection

pytestmark = pytest.mark.gpu

BASE = synth.CONFIGS["turbo_b8_t128k"].scaled(batch=2, hq=16, hkv=2, context=777)

CASES = [("hadamard", 16, 8, False), ("hadamard_plain", 16, 8, False), ("hadamard", 32, 8, False),
         ("hadamard", 16, 0, False), ("hadamard", 16, 8, True), ("hadamard_plain", 16, 8, True),
         ("hadamard", 32, 8, True), ("hadamard_plain", 32, 0, True)]


@pytest.mark.parametrize("rotation,hq,n_outlier,butterfly", CASES)
def test_structured_rotation_turbo_matches_oracle(rotation, hq, n_outlier, butterfly):
    cfg = BASE.scaled(hq=hq, n_outlier=n_outlier)
    print(f"[turbo {rotation}] hq={hq} outliers={n_outlier} butterfly={butterfly}", flush=True)
    g_proj = synth.gaussian_matrix(cfg.seed, 128, cfg.head_dim, stream=2)
    rev = rotation == "hadamard"
    consts = dict(rot=canonical_hadamard_rotation(cfg.head_dim, rev), proj=canonical_projection(g_proj))
    consts["levels"], consts["thresholds"] = canonical_codebook(2, cfg.head_dim)
    lib_consts = make_constants("turbo", cfg.head_dim, None, g_proj, rotation=rotation)
    kind = kvq.ROT_DENSE
    if butterfly:
        lib_consts.pop("rot")
        kind = kvq.ROT_HADAMARD_BITREV if rev else kvq.ROT_HADAMARD
    cache = PackedKVCache("turbo", cfg.batch, cfg.hkv, cfg.head_dim, cfg.context, device="cuda",
                          constants=lib_consts, rotation=kind)
    K, V = synth.make_kv(cfg, device="cuda")
    for t0, t1 in (((0, 600), (600, cfg.context)) if butterfly else ((0, 400), (400, cfg.context))):
        cache.append(K[:, :, t0:t1].contiguous(), V[:, :, t0:t1].contiguous(), t0)
    torch.cuda.synchronize()
    enc = oracle_encode(cfg, host64(K), host64(V), consts)
    assert_bytes_equal(gpu_buffers(cache), enc, f"turbo/{rotation}")
    q = synth.make_queries(cfg, device="cuda")
    lens = np.array([cfg.context, 301], dtype=np.int32)
    out = cache.decode(q, torch.from_numpy(lens).cuda(), softmax_scale(cfg)).cpu().numpy()
    ref = OA.decode_attention("turbo", enc, host64(q), lens, softmax_scale(cfg), cfg.hkv, consts)
    err = row_rel_err(out, ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= RTOL
