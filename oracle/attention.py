"""Oracle: attention over K/V gathered through a block table (float64).

Deep-dive page ("vLLM PagedAttention chuyên sâu ...", section "Cơ chế
PagedAttention"): for each query token the kernel (1) looks up the physical
blocks of the sequence in its block table, (2) gathers K and V from those
non-contiguous blocks, and (3) runs ordinary attention on what it gathered.
Ordinary attention here is softmax(q K^T * scale) V with the softmax taken over
all attended tokens.

Readings the pages leave open (stated once here):
  * a decode context length counts every attended token, including the token
    written in the same step;
  * grouped-query attention: query head h reads KV head h // (H / KVH);
  * prefill chunk (deep-dive page, section "Cơ chế của Chunked Prefill": chunks
    are processed in order and their KV accumulates in the cache): the chunk's
    n_q queries are the last n_q positions of the context, and query i sits at
    position L - n_q + i and attends to positions 0 .. L - n_q + i;
  * an empty context gives a zero output row.

Inputs are the *stored* values (bf16 widened exactly), so the oracle measures
only the kernel's own rounding.  No blocking, no online softmax: the plain
definition.
"""

from __future__ import annotations

import numpy as np

from .cache import read_key_page, read_value_page, to_f64


def gather_kv(k_cache, v_cache, block_table, context_len: int, kv_head: int, dtype: str):
    """Steps (1) and (2): K_s, V_s as float64 [L, head_dim], token t read from
    physical block block_table[t // block_size] at offset t % block_size (a
    whole page at a time, the last one cut at the context's end)."""
    block_size = k_cache.shape[3]
    L = int(context_len)
    ks, vs = [], []
    for j in range(-(-L // block_size)):
        phys = int(block_table[j])
        if phys < 0:
            raise ValueError(f"position {j * block_size} maps to an unallocated logical block")
        n = min(block_size, L - j * block_size)
        ks.append(read_key_page(k_cache, phys, kv_head)[:n])
        vs.append(read_value_page(v_cache, phys, kv_head)[:n])
    d = k_cache.shape[2] * k_cache.shape[4]
    if not ks:
        return np.zeros((0, d)), np.zeros((0, d))
    return to_f64(np.concatenate(ks), dtype), to_f64(np.concatenate(vs), dtype)


def softmax_weights(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """p_t = exp(s_t - max s) / sum_u exp(s_u - max s), s_t = scale * <q, K_t>."""
    s = float(scale) * (K @ q)
    e = np.exp(s - s.max())
    return e / e.sum()


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Step (3): sum_t p_t V_t (zero row for an empty context)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    return softmax_weights(q, K, scale) @ V


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
           pairs=None) -> np.ndarray:
    """Decode attention, one query token per sequence.

    q: [B, H, D] stored values; block_tables: [B, max_blocks] (-1 padded);
    context_lens: [B].  Returns float64 [B, H, D].  ``pairs`` optionally limits
    the work to a list of (sequence, head) outputs (others stay NaN).
    """
    q64 = to_f64(q, dtype)
    B, H, D = q64.shape
    kvh = k_cache.shape[1]
    group = H // kvh
    out = np.full((B, H, D), np.nan)
    want = None if pairs is None else {(int(s), int(h)) for s, h in pairs}
    for s in range(B):
        for g in range(kvh):
            heads = [h for h in range(g * group, (g + 1) * group)
                     if want is None or (s, h) in want]
            if not heads:
                continue
            K, V = gather_kv(k_cache, v_cache, block_tables[s], context_lens[s], g, dtype)
            for h in heads:
                out[s, h] = attend(q64[s, h], K, V, scale)
    return out


def decode_weights(q, k_cache, v_cache, block_table, context_len, head: int, num_kv_heads_group: int,
                   scale: float, dtype: str) -> np.ndarray:
    """The softmax weights of one (sequence, head) decode row."""
    g = head // num_kv_heads_group
    K, _ = gather_kv(k_cache, v_cache, block_table, context_len, g, dtype)
    return softmax_weights(to_f64(q, dtype), K, scale)


def prefill(q, k_cache, v_cache, block_tables, query_start_loc, context_lens, scale: float,
            dtype: str, rows=None) -> np.ndarray:
    """Causal chunked prefill over the paged cache.

    q: [Tq, H, D] packed by sequence, sequence s owning rows
    query_start_loc[s] .. query_start_loc[s+1]-1; context_lens[s] counts the
    cached tokens plus this chunk.  Returns float64 [Tq, H, D].  ``rows``
    optionally limits the work to a list of (query row, head) outputs.
    """
    q64 = to_f64(q, dtype)
    Tq, H, D = q64.shape
    kvh = k_cache.shape[1]
    group = H // kvh
    out = np.full((Tq, H, D), np.nan)
    want = None if rows is None else {(int(r), int(h)) for r, h in rows}
    B = len(context_lens)
    for s in range(B):
        r0, r1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
        n_q, L = r1 - r0, int(context_lens[s])
        for g in range(kvh):
            todo = [(r, h) for r in range(r0, r1) for h in range(g * group, (g + 1) * group)
                    if want is None or (r, h) in want]
            if not todo:
                continue
            K, V = gather_kv(k_cache, v_cache, block_tables[s], L, g, dtype)
            for r, h in todo:
                pos = L - n_q + (r - r0)
                out[r, h] = attend(q64[r, h], K[: pos + 1], V[: pos + 1], scale)
    return out


def prefill_rows(q, k_cache, v_cache, block_tables, query_start_loc, context_lens, scale: float,
                 dtype: str) -> np.ndarray:
    """The same outputs as ``prefill`` for every row, computed a (sequence,
    head) at a time in matrix form: S = scale * Q K^T over the chunk's rows,
    entries with key position > query position set to -inf, a softmax per row,
    then S V.  No blocking or online softmax: the definition with the rows of
    a (sequence, head) stacked."""
    q64 = to_f64(q, dtype)
    Tq, H, D = q64.shape
    kvh = k_cache.shape[1]
    group = H // kvh
    out = np.zeros((Tq, H, D))
    for s in range(len(context_lens)):
        r0, r1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
        n_q, L = r1 - r0, int(context_lens[s])
        if n_q == 0:
            continue
        pos = L - n_q + np.arange(n_q)                  # position of each chunk row
        masked = np.arange(L)[None, :] > pos[:, None]   # key after the query
        for g in range(kvh):
            K, V = gather_kv(k_cache, v_cache, block_tables[s], L, g, dtype)
            for h in range(g * group, (g + 1) * group):
                S = float(scale) * (q64[r0:r1, h] @ K.T)
                S[masked] = -np.inf
                P = np.exp(S - S.max(axis=1, keepdims=True))
                out[r0:r1, h] = (P / P.sum(axis=1, keepdims=True)) @ V
    return out


def decode_partitioned(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                       partition: int) -> np.ndarray:
    """Split-context decode of one row in float64: each partition of
    ``partition`` tokens yields (m_p, l_p, o_p) -- its max score, the sum of
    exp(s - m_p) and the normalised partial output -- and the partitions are
    merged with weights w_p = l_p * exp(m_p - max_p m_p):
    out = sum_p w_p o_p / sum_p w_p.  This is an exact rewrite of ``attend``;
    it exists to pin the merge algebra."""
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1])
    ms, ls, os_ = [], [], []
    for a in range(0, L, partition):
        s = float(scale) * (K[a:a + partition] @ q_row)
        m = s.max()
        e = np.exp(s - m)
        ms.append(m)
        ls.append(e.sum())
        os_.append((e @ V[a:a + partition]) / e.sum())
    M = max(ms)
    w = np.array([l * np.exp(m - M) for m, l in zip(ms, ls)])
    return (w[:, None] * np.stack(os_)).sum(0) / w.sum()
