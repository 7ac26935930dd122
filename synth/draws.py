"""Seeded random draws and workload scripts.

Every random quantity comes from its own counter-addressed stream
``numpy.random.Generator(PCG64(SeedSequence([seed, stream])))`` so that any
part of a workload can be regenerated lazily and in any order, on either side,
with identical values.

Stream numbering (per seed):
  0            structure: context lengths, suffix lengths, cached-prefix sizes
  1            the physical-block placement permutation (``free_order``)
  100 + j      K and V of the tokens appended by the j-th ``append`` op
  10**6 + k    the queries of batch step k
  2*10**6 + k  K and V of the tokens appended by extra decode step k >= 1
               (benchmarks that decode several steps in a row)

Values are N(0, 1) drawn in float32 (numpy's float32 normal sampler).  bf16
workloads store them rounded to bfloat16 with round-to-nearest-even, kept as
raw uint16 bit patterns.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

STREAM_STRUCTURE = 0
STREAM_PLACEMENT = 1
STREAM_APPEND0 = 100
STREAM_QUERY0 = 10**6
STREAM_EXTRA_STEP0 = 2 * 10**6


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bfloat16 bit patterns as uint16.  Inputs are finite draws, so
    no NaN special case is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _normal(g: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass(frozen=True)
class Spec:
    """Shapes and numeric type of one workload."""

    name: str
    kind: str  # "decode" or "prefill"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str  # "f32" or "bf16"
    partition: int = 0  # decode split-context partition size in tokens (0 = one pass)

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim), rounded to float32."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


@dataclass(frozen=True)
class Op:
    kind: str  # "new", "append", "fork"
    seq: int
    n: int = 0  # tokens appended ("append")
    parent: int = -1  # source sequence ("fork")
    stream: int = -1  # random stream of the appended tokens' K/V ("append")


@dataclass
class Script:
    """A workload: allocator operations, then one batch step.

    ``setup`` builds the cache history.  ``step`` holds the appends whose
    tokens belong to the timed batch step (the new decode token of every
    sequence, or every sequence's prefill chunk).  ``batch`` lists the
    sequences of the step in batch order, and ``query_lens[i]`` is the number
    of query tokens of ``batch[i]`` (1 for decode).
    """

    spec: Spec
    seed: int
    num_blocks: int
    free_order: np.ndarray  # int32 permutation of [0, num_blocks)
    setup: List[Op]
    step: List[Op]
    batch: List[int]
    query_lens: List[int]
    max_blocks_per_seq: int
    notes: dict = field(default_factory=dict)

    def ops(self):
        return list(self.setup) + list(self.step)

    def kv(self, op: Op):
        """(key, value) of an append op: arrays [n, num_kv_heads, head_dim]."""
        s = self.spec
        return kv_tokens(self.seed, op.stream, op.n, s.num_kv_heads, s.head_dim, s.dtype)

    def step_kv(self, step: int):
        """(key, value) [len(batch), KVH, D] of one more decode token per
        sequence, for decode step ``step`` >= 1 after the script's own step."""
        s = self.spec
        return kv_tokens(self.seed, STREAM_EXTRA_STEP0 + step, len(self.batch), s.num_kv_heads,
                         s.head_dim, s.dtype)

    def q(self, step: int = 0):
        """Queries of the batch step: [sum(query_lens), num_heads, head_dim]."""
        s = self.spec
        return queries(self.seed, step, int(sum(self.query_lens)), s.num_heads, s.head_dim, s.dtype)


def kv_tokens(seed: int, stream: int, n: int, num_kv_heads: int, head_dim: int, dtype: str):
    g = rng(seed, stream)
    k = _normal(g, (n, num_kv_heads, head_dim), dtype)
    v = _normal(g, (n, num_kv_heads, head_dim), dtype)
    return k, v


def queries(seed: int, step: int, n: int, num_heads: int, head_dim: int, dtype: str):
    return _normal(rng(seed, STREAM_QUERY0 + step), (n, num_heads, head_dim), dtype)


def placement(seed: int, num_blocks: int) -> np.ndarray:
    """Random order in which the pool hands out physical blocks."""
    return rng(seed, STREAM_PLACEMENT).permutation(num_blocks).astype(np.int32)


def _pool(needed: int, factor: float, minimum: Optional[int] = None) -> int:
    n = int(math.ceil(factor * needed))
    return max(n, minimum or 0, 1)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def decode_script(spec: Spec, lens: Sequence[int], seed: int, pool_factor: float = 1.25,
                  num_blocks: Optional[int] = None, growth: int = 64) -> Script:
    """Independent sequences decoding one token each.

    Sequence i holds ``lens[i] - 1`` history tokens; the step appends the
    token being decoded, so the step attends over ``lens[i]`` tokens.
    ``growth`` reserves table columns for later decode steps.
    """
    bs = spec.block_size
    lens = [int(x) for x in lens]
    needed = sum(_ceil_div(L, bs) for L in lens)
    nb = num_blocks if num_blocks is not None else _pool(needed, pool_factor)
    setup: List[Op] = []
    step: List[Op] = []
    j = 0
    for i, L in enumerate(lens):
        setup.append(Op("new", i))
        if L - 1 > 0:
            setup.append(Op("append", i, n=L - 1, stream=STREAM_APPEND0 + j))
            j += 1
    for i, L in enumerate(lens):
        if L > 0:
            step.append(Op("append", i, n=1, stream=STREAM_APPEND0 + j))
            j += 1
    mb = max(1, _ceil_div(max(lens) + growth, bs)) if lens else 1
    return Script(spec, seed, nb, placement(seed, nb), setup, step, list(range(len(lens))),
                  [1] * len(lens), mb, {"context_lens": lens})


def shared_prefix_script(spec: Spec, prompts: int, samples: int, prefix: int,
                         suffix_lens: Sequence[int], seed: int, pool_factor: float = 1.25,
                         growth: int = 64) -> Script:
    """Parallel sampling: every prompt's prefix is shared by its samples.

    Prompt p is sequence ``p*samples``; it appends the prefix, then forks
    ``samples-1`` children ``p*samples + j``.  Each sample then appends its
    private suffix history (``suffix - 1`` tokens, samples in index order),
    and the step appends every sample's decode token.
    """
    bs = spec.block_size
    suffix_lens = [int(x) for x in suffix_lens]
    assert len(suffix_lens) == prompts * samples
    full = prefix // bs
    needed = prompts * full + sum(_ceil_div(prefix + s, bs) - full for s in suffix_lens)
    nb = _pool(needed, pool_factor)
    setup: List[Op] = []
    step: List[Op] = []
    j = 0
    for p in range(prompts):
        root = p * samples
        setup.append(Op("new", root))
        setup.append(Op("append", root, n=prefix, stream=STREAM_APPEND0 + j))
        j += 1
        for c in range(1, samples):
            setup.append(Op("fork", root + c, parent=root))
    for p in range(prompts):
        for c in range(samples):
            s = p * samples + c
            n = suffix_lens[s] - 1
            if n > 0:
                setup.append(Op("append", s, n=n, stream=STREAM_APPEND0 + j))
                j += 1
    for s in range(prompts * samples):
        step.append(Op("append", s, n=1, stream=STREAM_APPEND0 + j))
        j += 1
    lens = [prefix + x for x in suffix_lens]
    mb = _ceil_div(max(lens) + growth, bs)
    return Script(spec, seed, nb, placement(seed, nb), setup, step, list(range(prompts * samples)),
                  [1] * (prompts * samples), mb,
                  {"context_lens": lens, "prefix": prefix, "prompts": prompts, "samples": samples})


def prefill_script(spec: Spec, cached: Sequence[int], chunk: int, seed: int,
                   pool_factor: float = 1.25) -> Script:
    """Chunked prefill: sequence i holds ``cached[i]`` tokens, the step appends
    a chunk of ``chunk`` tokens and runs them as queries."""
    bs = spec.block_size
    cached = [int(x) for x in cached]
    needed = sum(_ceil_div(c + chunk, bs) for c in cached)
    nb = _pool(needed, pool_factor)
    setup: List[Op] = []
    step: List[Op] = []
    j = 0
    for i, c in enumerate(cached):
        setup.append(Op("new", i))
        if c > 0:
            setup.append(Op("append", i, n=c, stream=STREAM_APPEND0 + j))
            j += 1
    for i in range(len(cached)):
        step.append(Op("append", i, n=chunk, stream=STREAM_APPEND0 + j))
        j += 1
    lens = [c + chunk for c in cached]
    mb = _ceil_div(max(lens), bs)
    return Script(spec, seed, nb, placement(seed, nb), setup, step, list(range(len(cached))),
                  [chunk] * len(cached), mb, {"context_lens": lens, "cached": cached})


def mixed_script(spec: Spec, cached: Sequence[int], chunk: int, decode_lens: Sequence[int],
                 seed: int, pool_factor: float = 1.25) -> Script:
    """A batch mixing prefill chunks and decode tokens.

    Sequences 0 .. len(cached)-1 hold ``cached[i]`` tokens and the step
    appends a chunk of ``chunk`` tokens (its query rows); sequences after them
    hold ``decode_lens[j] - 1`` tokens and the step appends one token (one
    query row).  ``spec.kind`` is "prefill": a decode token is a chunk of
    one."""
    bs = spec.block_size
    cached = [int(x) for x in cached]
    decode_lens = [int(x) for x in decode_lens]
    P = len(cached)
    needed = (sum(_ceil_div(c + chunk, bs) for c in cached)
              + sum(_ceil_div(L, bs) for L in decode_lens))
    nb = _pool(needed, pool_factor)
    setup: List[Op] = []
    step: List[Op] = []
    j = 0
    hist = cached + [L - 1 for L in decode_lens]
    for i, c in enumerate(hist):
        setup.append(Op("new", i))
        if c > 0:
            setup.append(Op("append", i, n=c, stream=STREAM_APPEND0 + j))
            j += 1
    qlens = [chunk] * P + [1] * len(decode_lens)
    for i, n in enumerate(qlens):
        step.append(Op("append", i, n=n, stream=STREAM_APPEND0 + j))
        j += 1
    lens = [c + chunk for c in cached] + decode_lens
    mb = _ceil_div(max(lens), bs)
    return Script(spec, seed, nb, placement(seed, nb), setup, step, list(range(len(lens))),
                  qlens, mb, {"context_lens": lens, "cached": cached, "num_prefill": P,
                              "chunk": chunk})
