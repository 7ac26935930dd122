"""Seeded synthetic inputs for the paged-attention workloads.

This package draws random numbers and lays out the *structure* of a workload:
which sequences exist, in which order they are created, how many tokens each
one appends, which sequences fork from which, and the K/V/Q values of every
token.  It holds none of the method's arithmetic -- no block tables, no slot
numbers, no cache layout, no attention.  The oracle side and the HIP side each
execute the scripts produced here with their own block allocator and their own
cache writes, so the only thing they share is the random draws.
"""

from .draws import (
    Op,
    Script,
    Spec,
    bf16_bits_from_f32,
    kv_tokens,
    queries,
    decode_script,
    shared_prefix_script,
    prefill_script,
    mixed_script,
)
from .configs import CONFIGS, config_script
from .prompts import multi_turn_requests, prefix_kv, prompt_queries

__all__ = [
    "Op",
    "Script",
    "Spec",
    "bf16_bits_from_f32",
    "kv_tokens",
    "queries",
    "decode_script",
    "shared_prefix_script",
    "prefill_script",
    "mixed_script",
    "CONFIGS",
    "config_script",
    "multi_turn_requests",
    "prefix_kv",
    "prompt_queries",
]
