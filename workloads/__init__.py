"""Synthetic attention workloads: sizes/flags (configs) and seeded inputs (gen).

Shared by the oracle-side tests and the GPU-side tests and benchmark; it holds
no attention arithmetic.
"""
from . import configs, gen  # noqa: F401
