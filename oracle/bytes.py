"""Bytes stored per token.

Page "TurboQuant vs OSCAR vs EpiCache", section on the KV-cache memory
bottleneck: a decoder keeps one key and one value vector per token, per layer,
per KV head, so the per-token size is layers x KV heads x head dim x 2 tensors
x bytes per element (0.31 MB for a 70B-class model in BF16).  For a packed
format the element bytes become the packed codes plus the metadata stored for
that token; metadata shared by a group of tokens (KIVI key scale/zero, one per
32 tokens) is divided evenly over the group.
"""


def per_token_head(fmt: str, d: int, rope_dim: int = 0, m: int = 128) -> float:
    """Bytes per token per KV head (per token for the shared latent)."""
    if fmt == "bf16":
        return 2 * d * 2                       # K and V, 2 bytes each
    if fmt == "fp4":
        return 2 * (d // 2 + 2 * (d // 16))    # nibbles + one bf16 scale per 16, for K and V
    if fmt == "kivi2":
        k = d // 4 + (4 + 4) * d / 32          # codes + fp32 scale/zero per channel per 32 tokens
        v = d // 4 + (4 + 4) * (d // 32)       # codes + fp32 scale/zero per 32 channels
        return k + v
    if fmt == "turbo":
        k = d // 4 + m // 8 + 2 + 2            # LM codes + sketch + fp16 norm + fp16 residual norm
        v = d // 4 + 2                         # LM codes + fp16 norm
        return k + v
    if fmt == "qjl1":
        return (m // 8 + 2) + (d // 2 + 2 * (d // 16))
    if fmt == "latent":
        return d // 2 + 2 * (d // 16) + 2 * rope_dim
    raise ValueError(fmt)


def bytes_per_token(fmt: str, num_kv_heads: int, d: int, num_layers: int, rope_dim: int = 0,
                    m: int = 128) -> int:
    v = num_layers * num_kv_heads * per_token_head(fmt, d, rope_dim, m)
    assert float(v).is_integer()
    return int(v)
