"""Seeded synthetic inputs for the low-bit KV-cache tests, bench and smoke run.

This package only draws random numbers and lays them out in the shapes of the
five workloads.  It holds none of the quantisation or attention arithmetic:
the HIP library and the CPU oracle each do their own, and both receive the
tensors made here.

Random numbers that the methods themselves draw (the Gaussian matrix whose QR
factor is the TurboQuant rotation, the Gaussian QJL projection) are drawn here
as plain float64 arrays and handed to both sides as inputs.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    gaussian_matrix,
    make_kv,
    make_indexer_scores,
    make_latent,
    make_queries,
    outlier_channels,
    seq_lens_for,
)
