"""The five workload shapes, as data.

Shapes come from the pages: the 70B-class cache geometry (80 layers x 8 KV
heads x 128 channels, page "TurboQuant vs OSCAR vs EpiCache", section on the
KV-cache memory bottleneck), 128K / 1M contexts (same section), key-only fixed
outlier channels (same page, KIVI paragraph of "quantization frontiers") and the
512-wide latent plus 64-wide RoPE key shared by all heads (page "How
DeepSeek-V4.1-Flash cut KV-cache storage by 4x via CSA2", CSA2 section).
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    fmt: str            # "kivi2" | "fp4" | "turbo" | "qjl1" | "latent"
    batch: int
    hq: int             # query heads
    hkv: int            # KV heads (1 for the shared latent)
    head_dim: int       # key/value width (latent width for "latent")
    rope_dim: int       # bf16 RoPE key width ("latent" only)
    context: int        # cached tokens per sequence seen by the decode step
    in_dtype: str       # "f32" | "bf16" for K/V/latent inputs
    q_dtype: str        # "f32" | "bf16"
    n_outlier: int      # fixed outlier key channels per KV head
    outlier_scale: float
    append_new: int     # tokens appended in bulk inside the timed step (0: none)
    seed: int

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def key_width(self) -> int:
        return self.head_dim + self.rope_dim

    def scaled(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # 1 seq, 4 q / 2 KV heads, d=64, 256 tokens, fp32 Q/K/V, 4 outlier key channels x20.
    "kivi2_tiny": Config("kivi2_tiny", "kivi2", 1, 4, 2, 64, 0, 256, "f32", "f32", 4, 20.0, 0, 101),
    # 8B-class layer: 32 q / 8 KV heads, d=128, batch 16, 32K context, 8 outlier key channels x15.
    "fp4_b16_t32k": Config("fp4_b16_t32k", "fp4", 16, 32, 8, 128, 0, 32768, "bf16", "bf16", 8, 15.0, 0, 102),
    # 70B-class layer: 64 q / 8 KV heads, d=128, batch 8, 128K context, 8 outlier key channels x20.
    "turbo_b8_t128k": Config("turbo_b8_t128k", "turbo", 8, 64, 8, 128, 0, 131072, "bf16", "bf16", 8, 20.0, 0, 103),
    # 1-bit keys at 1M context, batch 1, 32 q / 8 KV heads; 32768-token bulk append.
    "qjl1_b1_t1m": Config("qjl1_b1_t1m", "qjl1", 1, 32, 8, 128, 0, 1048576, "bf16", "bf16", 0, 1.0, 32768, 104),
    # Shared latent: 128 q heads over one 512-wide FP4 latent + 64-wide bf16 RoPE key, batch 64, 64K.
    "latent_b64_t64k": Config("latent_b64_t64k", "latent", 64, 128, 1, 512, 64, 65536, "bf16", "bf16", 0, 1.0, 0, 105),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]
