"""Seeded synthetic inputs for single-query decode attention.

This package builds the query, KV-cache and block-table inputs that both the
HIP library and the CPU oracle consume.  It holds no part of the attention
arithmetic itself: it draws Gaussian values, rounds them to the storage dtype,
lays caches out, and plants score structure into keys.  See `synth` for the
recipes.
"""
from .synth import (  # noqa: F401
    DenseCase, PagedCase, UnifiedCase, FfdCase,
    dense_case, paged_case, unified_case, ffd_case, multi_case,
    config_case, CONFIGS,
)
