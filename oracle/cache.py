"""Oracle: the paged KV-cache layout, the cache write and the block copy.

The deep-dive page ("vLLM PagedAttention chuyên sâu ...", section "Tương tự
phân trang bộ nhớ ảo") splits each sequence's KV cache into logical blocks of a
fixed number of tokens, each stored in a fixed-size physical block anywhere in
GPU memory.  The pages do not fix the byte layout inside a physical block; this
library's documented layout is (X = 16 bytes / element size: 8 for bf16,
4 for fp32):

  k_cache[num_blocks][num_kv_heads][head_dim / X][block_size][X]
  v_cache[num_blocks][num_kv_heads][head_dim][block_size]

i.e. key element (block b, kv head g, in-block offset o, dim d) lives at
k_cache[b, g, d // X, o, d % X] and the value element at v_cache[b, g, d, o].

A slot is a flat token position in the pool: slot = block * block_size + offset.
Slot mapping of a sequence position (same page, same section: the block table
maps logical to physical block indices) is computed by ``AllocModel``.

Everything here is exact data movement: arrays are handled as raw bit patterns
(uint16 for bf16, uint32 views for fp32) so results are compared bit for bit.
"""

from __future__ import annotations

import numpy as np


def chunk_elems(dtype: str) -> int:
    """X: elements per 16-byte chunk of the key layout."""
    return {"f32": 4, "bf16": 8}[dtype]


def storage_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16}[dtype]


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float64: bf16 bits are widened exactly (bits << 16)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def empty_cache(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int, dtype: str,
                poison: int | None = None):
    """Fresh (k_cache, v_cache) in the documented layout, filled with a bit
    pattern (default all-ones bits: a NaN in both fp32 and bf16)."""
    x = chunk_elems(dtype)
    assert head_dim % x == 0
    st = storage_dtype(dtype)
    kshape = (num_blocks, num_kv_heads, head_dim // x, block_size, x)
    vshape = (num_blocks, num_kv_heads, head_dim, block_size)
    if st is np.uint16:
        fill = 0xFFFF if poison is None else poison
        return np.full(kshape, fill, np.uint16), np.full(vshape, fill, np.uint16)
    fill = 0xFFFFFFFF if poison is None else poison
    k = np.full(kshape, fill, np.uint32).view(np.float32)
    v = np.full(vshape, fill, np.uint32).view(np.float32)
    return k, v


def read_key(k_cache: np.ndarray, block: int, head: int, offset: int) -> np.ndarray:
    """The key row [head_dim] stored at (block, head, offset)."""
    return k_cache[block, head, :, offset, :].reshape(-1)


def read_value(v_cache: np.ndarray, block: int, head: int, offset: int) -> np.ndarray:
    """The value row [head_dim] stored at (block, head, offset)."""
    return v_cache[block, head, :, offset]


def read_key_page(k_cache: np.ndarray, block: int, head: int) -> np.ndarray:
    """All key rows of one (block, head) page: [block_size, head_dim], row o
    being read_key(k_cache, block, head, o)."""
    page = k_cache[block, head]                      # [head_dim / X, block_size, X]
    return page.transpose(1, 0, 2).reshape(page.shape[1], -1)


def read_value_page(v_cache: np.ndarray, block: int, head: int) -> np.ndarray:
    """All value rows of one (block, head) page: [block_size, head_dim], row o
    being read_value(v_cache, block, head, o)."""
    return v_cache[block, head].T


def reshape_and_cache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray,
                      v_cache: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Write new tokens' K/V into their cache slots, in place.

    key, value: [T, num_kv_heads, head_dim]; slot_mapping: [T] int64.
    Token i goes to block slot // block_size at offset slot % block_size, for
    every KV head.  A negative slot means "no write" (a padding token).
    Growing a sequence writes into newly mapped physical blocks without moving
    the old ones (deep-dive page, section "Tương tự phân trang bộ nhớ ảo",
    dynamic resizing).
    """
    block_size = k_cache.shape[3]
    x = k_cache.shape[4]
    num_kv_heads, head_dim = key.shape[1], key.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        b, o = int(slot) // block_size, int(slot) % block_size
        # every KV head of token i at once: head g, chunk c, element e
        k_cache[b, :, :, o, :] = key[i].reshape(num_kv_heads, head_dim // x, x)
        v_cache[b, :, :, o] = value[i]


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> None:
    """Copy-on-write block copies, in place: for each (src, dst) pair, in
    order, the whole physical block src (all KV heads, all offsets) is copied
    to dst, for K and for V (deep-dive page, section "Cơ chế APC", item 3:
    a sequence that diverges from shared blocks copies them and goes on alone).
    """
    for src, dst in pairs:
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]
