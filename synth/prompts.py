"""Seeded token-id prompts for prefix caching, and K/V that depend on the
token prefix.

A language model's K/V for position p is a function of the tokens 0..p; the
synthetic stand-in here draws them from a stream addressed by a 64-bit chained
hash of that prefix, so equal prefixes get equal K/V and any difference in an
earlier token changes every later position.  No model, vocabulary or dataset
is involved: token ids are small random integers.

Streams (per seed): 3*10**6 structure of the prompts, 4*10**6 the queries.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .draws import _normal, rng

STREAM_PROMPTS = 3 * 10**6
STREAM_PROMPT_Q = 4 * 10**6
_MASK = (1 << 64) - 1


def _mix(h: int, t: int) -> int:
    """splitmix64 finaliser over (h, token): the prefix hash chain."""
    z = (h ^ ((t + 0x9E3779B97F4A7C15) & _MASK)) & _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def prefix_hashes(tokens: Sequence[int]) -> List[int]:
    """hash of tokens[0..p] for every p."""
    out, h = [], 0
    for t in tokens:
        h = _mix(h, int(t))
        out.append(h)
    return out


def prefix_kv(seed: int, tokens: Sequence[int], start: int, num_kv_heads: int, head_dim: int,
              dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """K and V [len(tokens) - start, num_kv_heads, head_dim] of positions
    start.. of a sequence with these token ids."""
    hs = prefix_hashes(tokens)
    n = len(tokens) - start
    k = np.empty((n, num_kv_heads, head_dim), np.uint16 if dtype == "bf16" else np.float32)
    v = np.empty_like(k)
    for i in range(n):
        h = hs[start + i]
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, h >> 32, h & 0xFFFFFFFF])))
        k[i] = _normal(g, (num_kv_heads, head_dim), dtype)
        v[i] = _normal(g, (num_kv_heads, head_dim), dtype)
    return k, v


def multi_turn_requests(seed: int, dialogues: int, turns: int, system_len: int, user_len: int,
                        answer_len: int, vocab: int = 32000):
    """Chat requests with a common system prompt and growing histories.

    Dialogue d's turn t prompt is the system prompt, then turns 0..t-1's user
    text and answer, then turn t's user text.  Returns a list, in arrival
    order (turn by turn, dialogues interleaved), of (dialogue, turn, prompt
    token ids, answer token ids).
    """
    g = rng(seed, STREAM_PROMPTS)
    system = g.integers(0, vocab, size=system_len).tolist()
    hist = [list(system) for _ in range(dialogues)]
    out = []
    for t in range(turns):
        for d in range(dialogues):
            user = g.integers(0, vocab, size=user_len).tolist()
            answer = g.integers(0, vocab, size=answer_len).tolist()
            prompt = hist[d] + user
            out.append((d, t, prompt, answer))
            hist[d] = prompt + answer
    return out


def prompt_queries(seed: int, n: int, num_heads: int, head_dim: int, dtype: str) -> np.ndarray:
    return _normal(rng(seed, STREAM_PROMPT_Q), (n, num_heads, head_dim), dtype)
