"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package draws random numbers and rounds them to the storage dtype.
It holds none of the attention method's arithmetic.
"""
from .inputs import CONFIGS, config, make, ragged, round_bf16, shrink  # noqa: F401
