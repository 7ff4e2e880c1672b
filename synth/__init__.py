"""Seeded synthetic workloads for the exit-and-KV-fill step.

This package only draws and lays out inputs (hidden states, router and
K/V weights, their int4 storage form, cache slots). It holds none of the
step's arithmetic: no cosine, router, compaction, projection or ridge solve.
Both the GPU tests/benchmark and the oracle-based checks take their inputs
from here, so the two sides always see identical values.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
