"""Seeded synthetic inputs for the head-aware sparse decode workloads.

This package is shared by both sides of every parity check: it draws
weights, queries, key/value caches, dominant-chunk sets and planted
structure from a counter-based generator (Philox4x32-10), on the host for
slices the CPU oracle needs and on the device for whole caches.  It holds
none of the attention method's arithmetic.
"""
from .recipe import CONFIGS, Config, get_config  # noqa: F401
