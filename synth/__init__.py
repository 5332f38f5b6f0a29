"""Seeded synthetic KV-cache inputs.

This package only makes inputs: planted-Tucker caches with noise and outlier
channels, cast to the storage dtype, plus the named workload shapes.  It holds
none of the compressor's arithmetic; both the CPU oracle and the HIP path read
their inputs from here.
"""
from .caches import (  # noqa: F401
    CacheConfig,
    CONFIGS,
    Item,
    config,
    item_specs,
    make_item,
    make_items,
    budget_for_ratio,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    iter_raw_parallel,
)
