"""The five benchmark workloads, as seeded scripts.

  tiny_decode_f32      4 sequences, contexts {30, 50, 17, 64}, 4 heads, head_dim 64,
                       fp32, 32-block pool placed by a random permutation
  decode_bf16          64 sequences, 32 heads = 32 KV heads, head_dim 128,
                       contexts uniform in [512, 2048], pool 1.25x the blocks needed
  gqa_decode_bf16      256 sequences, 64 query heads over 8 KV heads, head_dim 128,
                       contexts log-uniform in [128, 8192], 512-token partitions
  shared_prefix_bf16   32 prompts x 8 samples, 32 heads, head_dim 128, a 1024-token
                       prefix shared by each prompt's samples, suffixes uniform in [1, 256]
  chunked_prefill_bf16 16 sequences, 512-token causal query chunks after 0..3584
                       cached tokens (multiples of 16), 32 heads, head_dim 128

All use block_size 16, and the bf16 decode workloads 512-token split-context
partitions (stated for GQA; for the others the fastest measured of 0, 256,
512 and 1024 that still splits their longer contexts).
``shared_prefix_cow_bf16`` is the same as
``shared_prefix_bf16`` with a 1020-token prefix, so that the last shared block
is partially filled and every diverging sample but the last copies it first.
"""

from __future__ import annotations

import math

import numpy as np

from .draws import (STREAM_STRUCTURE, Script, Spec, decode_script, prefill_script, rng,
                    shared_prefix_script)

BS = 16

SPECS = {
    "tiny_decode_f32": Spec("tiny_decode_f32", "decode", 4, 4, 64, BS, "f32", partition=0),
    "decode_bf16": Spec("decode_bf16", "decode", 32, 32, 128, BS, "bf16", partition=512),
    "gqa_decode_bf16": Spec("gqa_decode_bf16", "decode", 64, 8, 128, BS, "bf16", partition=512),
    "shared_prefix_bf16": Spec("shared_prefix_bf16", "decode", 32, 32, 128, BS, "bf16", partition=512),
    "shared_prefix_cow_bf16": Spec("shared_prefix_cow_bf16", "decode", 32, 32, 128, BS, "bf16",
                                   partition=512),
    "chunked_prefill_bf16": Spec("chunked_prefill_bf16", "prefill", 32, 32, 128, BS, "bf16"),
}

CONFIGS = ["tiny_decode_f32", "decode_bf16", "gqa_decode_bf16", "shared_prefix_bf16",
           "chunked_prefill_bf16"]

DEFAULT_SEED = {name: i + 1 for i, name in enumerate(CONFIGS)}
DEFAULT_SEED["shared_prefix_cow_bf16"] = 4


def log_uniform_lengths(g: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    x = np.exp(g.uniform(math.log(lo), math.log(hi), size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def config_script(name: str, seed: int | None = None, scale_down: int = 1) -> Script:
    """Script of a named workload.

    ``scale_down`` > 1 divides the number of sequences (and prompts) by that
    factor, keeping every per-sequence distribution, for quick parity runs.
    """
    spec = SPECS[name]
    seed = DEFAULT_SEED[name] if seed is None else int(seed)
    g = rng(seed, STREAM_STRUCTURE)
    sd = max(1, int(scale_down))
    if name == "tiny_decode_f32":
        return decode_script(spec, [30, 50, 17, 64], seed, num_blocks=32, growth=0)
    if name == "decode_bf16":
        lens = g.integers(512, 2048, size=max(1, 64 // sd), endpoint=True)
        return decode_script(spec, lens, seed)
    if name == "gqa_decode_bf16":
        lens = log_uniform_lengths(g, max(1, 256 // sd), 128, 8192)
        return decode_script(spec, lens, seed)
    if name in ("shared_prefix_bf16", "shared_prefix_cow_bf16"):
        prompts, samples = max(1, 32 // sd), 8
        prefix = 1024 if name == "shared_prefix_bf16" else 1020
        suffix = g.integers(1, 256, size=prompts * samples, endpoint=True)
        return shared_prefix_script(spec, prompts, samples, prefix, suffix, seed)
    if name == "chunked_prefill_bf16":
        cached = BS * g.integers(0, 3584 // BS, size=max(1, 16 // sd), endpoint=True)
        return prefill_script(spec, cached, 512, seed)
    raise KeyError(name)
