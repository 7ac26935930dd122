"""Torch-facing binding of libpa's kernel entry points.

Same names as the C ABI.  Each function validates shapes/dtypes on the host,
then passes raw device pointers and the current HIP stream to libpa.  Torch
only provides device memory and the stream; all work runs in libpa's HIP
kernels.  ``check_device_args=True`` additionally copies block tables and
context lengths to the host and verifies the preconditions libpa does not
check on the device (useful in tests; it synchronises).
"""

from __future__ import annotations

import numpy as np
import torch

from ._lib import PA_BF16, PA_DECODE_FIND_SHARED, PA_DECODE_STREAM_KV, PA_F32, check, lib

BLOCK_SIZE = 16
_DT = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}


def chunk_elems(dtype: torch.dtype) -> int:
    """X: elements per 16-byte chunk of the key layout."""
    return 16 // torch.tensor([], dtype=dtype).element_size()


def new_kv_cache(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 device="cuda", block_size: int = BLOCK_SIZE):
    """Uninitialised (k_cache, v_cache) in libpa's layout:
    k_cache [num_blocks, num_kv_heads, head_dim // X, block_size, X],
    v_cache [num_blocks, num_kv_heads, head_dim, block_size]."""
    x = chunk_elems(dtype)
    k = torch.empty((num_blocks, num_kv_heads, head_dim // x, block_size, x), dtype=dtype, device=device)
    v = torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=dtype, device=device)
    return k, v


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _flags(stream_kv: bool, find_shared: bool = False) -> int:
    return (PA_DECODE_STREAM_KV if stream_kv else 0) | (PA_DECODE_FIND_SHARED if find_shared else 0)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _arg(dev: torch.device, name: str, t, dtype=None, contiguous: bool = True):
    """Check one tensor argument before its address goes to libpa: a tensor on
    the caches' device, of the given dtype, contiguous (with contiguous=False,
    the caller's stride checks apply).  A host tensor's address would reach a
    kernel as a device address."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}; it must be on the caches' device {dev}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    if v_cache.device != k_cache.device:
        raise ValueError("k_cache and v_cache must be on one device")
    if k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("k_cache must be 5-D and v_cache 4-D (libpa layout)")
    nb, kvh, dx, bs, x = k_cache.shape
    d = dx * x
    if tuple(v_cache.shape) != (nb, kvh, d, bs):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} does not match k_cache {tuple(k_cache.shape)}")
    if x != chunk_elems(k_cache.dtype) or v_cache.dtype != k_cache.dtype:
        raise ValueError("cache dtype/chunk mismatch")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    return nb, kvh, d, bs


def _check_tables(block_tables, context_lens, num_blocks, block_size):
    bt = block_tables.cpu().numpy()
    lens = context_lens.cpu().numpy()
    mb = bt.shape[1]
    for s, L in enumerate(lens):
        if L < 0 or L > mb * block_size:
            raise ValueError(f"context_lens[{s}]={L} outside [0, {mb * block_size}]")
        used = bt[s, : -(-int(L) // block_size)]
        if used.size and (used.min() < 0 or used.max() >= num_blocks):
            raise ValueError(f"block_tables[{s}] names a block outside the pool")


def pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, check_device_args=False):
    nb, kvh, d, bs = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _arg(dev, "key", key, contiguous=False)
    _arg(dev, "value", value, contiguous=False)
    _arg(dev, "slot_mapping", slot_mapping, torch.int64)
    T = key.shape[0]
    if key.shape[1:] != (kvh, d) or value.shape[1:] != (kvh, d) or value.shape[0] != T:
        raise ValueError("key/value must be [T, num_kv_heads, head_dim]")
    if key.dtype != k_cache.dtype or value.dtype != k_cache.dtype:
        raise TypeError("key/value dtype must match the cache")
    if key.stride(2) != 1 or key.stride(1) != d or value.stride(2) != 1 or value.stride(1) != d:
        raise ValueError("key/value heads must be contiguous rows")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,) or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int64 [T]")
    if check_device_args and T:
        s = slot_mapping.cpu().numpy()
        s = s[s >= 0]
        if s.size and (s.max() >= nb * bs or len(np.unique(s)) != s.size):
            raise ValueError("slots out of range or repeated")
    check("pa_reshape_and_cache", lib().pa_reshape_and_cache(
        key.data_ptr(), value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        slot_mapping.data_ptr(), T, key.stride(0), value.stride(0), kvh, d, bs, nb,
        _dtype(k_cache), _stream(k_cache)))


def pa_copy_blocks(k_cache, v_cache, pairs):
    nb, kvh, d, bs = _cache_dims(k_cache, v_cache)
    _arg(k_cache.device, "pairs", pairs, torch.int32)
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2 or not pairs.is_contiguous():
        raise ValueError("pairs must be contiguous int32 [n, 2]")
    check("pa_copy_blocks", lib().pa_copy_blocks(
        k_cache.data_ptr(), v_cache.data_ptr(), pairs.data_ptr(), pairs.shape[0], kvh, d, bs, nb,
        _dtype(k_cache), _stream(k_cache)))


def pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition,
                              find_shared: bool = False) -> int:
    """Workspace of pa_decode; ``find_shared``: with PA_DECODE_FIND_SHARED."""
    return int(lib().pa_decode_workspace_bytes_flags(num_seqs, num_heads, head_dim,
                                                     max_context_len, partition,
                                                     _flags(False, find_shared)))


def decode_workspace(num_seqs, num_heads, head_dim, max_context_len, partition, device="cuda",
                     find_shared: bool = False):
    n = pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition,
                                  find_shared)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, partition: int,
              max_context_len: int, workspace=None, check_device_args=False,
              stream_kv: bool = False, find_shared: bool = False):
    """``stream_kv``: PA_DECODE_STREAM_KV, for calls in which no block is read
    by two sequences; ``find_shared``: PA_DECODE_FIND_SHARED, the call finds
    prefix groups itself and reads their shared pages once (see
    include/pa.h)."""
    nb, kvh, d, bs = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _arg(dev, "out", out)
    _arg(dev, "q", q)
    _arg(dev, "block_tables", block_tables, torch.int32)
    _arg(dev, "context_lens", context_lens, torch.int32)
    if workspace is not None:
        _arg(dev, "workspace", workspace)
    B, H = q.shape[0], q.shape[1]
    if q.shape != (B, H, d) or out.shape != q.shape or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q/out must be contiguous [B, H, head_dim]")
    if q.dtype != k_cache.dtype or out.dtype != q.dtype:
        raise TypeError("q/out dtype must match the cache")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B \
            or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    if check_device_args:
        _check_tables(block_tables, context_lens, nb, bs)
        if int(context_lens.max()) > max_context_len:
            raise ValueError("max_context_len below a context length")
    need = pa_decode_workspace_bytes(B, H, d, max_context_len, partition, find_shared)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("pa_decode", lib().pa_decode(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(), B, H, kvh, d, bs,
        nb, float(scale), int(partition), int(max_context_len), wptr, wbytes, _dtype(q),
        _flags(stream_kv, find_shared), _stream(q)))


def pa_decode_no_alloc(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                       partition: int, max_context_len: int, stream_kv: bool = False,
                       find_shared: bool = False):
    """pa_decode with the partials in the library's own device array: no
    workspace, no allocation (see include/pa.h for the size limit and the rule
    that overlapping calls on one GPU race)."""
    nb, kvh, d, bs = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _arg(dev, "out", out)
    _arg(dev, "q", q)
    _arg(dev, "block_tables", block_tables, torch.int32)
    _arg(dev, "context_lens", context_lens, torch.int32)
    B, H = q.shape[0], q.shape[1]
    if q.shape != (B, H, d) or out.shape != q.shape:
        raise ValueError("q/out must be [B, H, head_dim]")
    if q.dtype != k_cache.dtype or out.dtype != q.dtype:
        raise TypeError("q/out dtype must match the cache")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    check("pa_decode_no_alloc", lib().pa_decode_no_alloc(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(), B, H, kvh, d, bs,
        nb, float(scale), int(partition), int(max_context_len), _dtype(q),
        _flags(stream_kv, find_shared), _stream(q)))


def pa_prefix_plan(block_tables, context_lens, max_members: int = 8, min_prefix: int = 256,
                   block_size: int = BLOCK_SIZE):
    """Prefix groups of a batch (host arrays or tensors; runs on the host).

    Returns (groups int32 [num_groups, 3] = (first sequence, members, prefix
    tokens), seq_prefix_lens int32 [num_seqs], max_prefix_len)."""
    bt = np.ascontiguousarray(np.asarray(block_tables.cpu() if torch.is_tensor(block_tables)
                                         else block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(context_lens.cpu() if torch.is_tensor(context_lens)
                                           else context_lens, dtype=np.int32))
    if bt.ndim != 2 or lens.shape != (bt.shape[0],):
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    B = bt.shape[0]
    groups = np.zeros((max(B, 1), 3), dtype=np.int32)
    pre = np.zeros(max(B, 1), dtype=np.int32)
    ng = np.zeros(1, dtype=np.int32)
    mp = np.zeros(1, dtype=np.int32)
    check("pa_prefix_plan", lib().pa_prefix_plan(
        bt.ctypes.data, bt.shape[1], lens.ctypes.data, B, int(block_size), int(max_members),
        int(min_prefix), groups.ctypes.data, pre.ctypes.data, ng.ctypes.data, mp.ctypes.data))
    return groups[: int(ng[0])].copy(), pre[:B].copy(), int(mp[0])


def pa_decode_shared_prefix_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                            max_prefix_len, partition) -> int:
    return int(lib().pa_decode_shared_prefix_workspace_bytes(
        num_seqs, num_heads, head_dim, max_context_len, max_prefix_len, partition))


def pa_decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                            partition: int, max_context_len: int, prefix_groups,
                            seq_prefix_lens, max_prefix_len: int, workspace=None,
                            check_device_args=False, stream_kv: bool = False):
    """pa_decode with prefix groups (device int32 tensors [G, 3] and [B], as
    pa_prefix_plan returns them)."""
    nb, kvh, d, bs = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _arg(dev, "out", out)
    _arg(dev, "q", q)
    _arg(dev, "block_tables", block_tables, torch.int32)
    _arg(dev, "context_lens", context_lens, torch.int32)
    _arg(dev, "prefix_groups", prefix_groups, torch.int32)
    _arg(dev, "seq_prefix_lens", seq_prefix_lens, torch.int32)
    if workspace is not None:
        _arg(dev, "workspace", workspace)
    B, H = q.shape[0], q.shape[1]
    if q.shape != (B, H, d) or out.shape != q.shape or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q/out must be contiguous [B, H, head_dim]")
    if q.dtype != k_cache.dtype or out.dtype != q.dtype:
        raise TypeError("q/out dtype must match the cache")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B \
            or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    ng = int(prefix_groups.shape[0])
    if prefix_groups.dtype != torch.int32 or prefix_groups.dim() != 2 or prefix_groups.shape[1] != 3 \
            or not prefix_groups.is_contiguous():
        raise ValueError("prefix_groups must be contiguous int32 [num_groups, 3]")
    if seq_prefix_lens.dtype != torch.int32 or seq_prefix_lens.shape != (B,):
        raise ValueError("seq_prefix_lens must be int32 [B]")
    if check_device_args:
        _check_tables(block_tables, context_lens, nb, bs)
        if int(context_lens.max()) > max_context_len:
            raise ValueError("max_context_len below a context length")
        _check_groups(block_tables.cpu().numpy(), context_lens.cpu().numpy(),
                      prefix_groups.cpu().numpy(), seq_prefix_lens.cpu().numpy(), max_prefix_len, bs)
    need = pa_decode_shared_prefix_workspace_bytes(B, H, d, max_context_len, max_prefix_len,
                                                   partition)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("pa_decode_shared_prefix", lib().pa_decode_shared_prefix(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(), B, H, kvh, d, bs,
        nb, float(scale), int(partition), int(max_context_len),
        prefix_groups.data_ptr() if ng else None, ng,
        seq_prefix_lens.data_ptr(), int(max_prefix_len), wptr, wbytes, _dtype(q),
        _flags(stream_kv), _stream(q)))


def _check_groups(bt, lens, groups, pre, max_prefix_len, bs):
    covered = np.zeros(bt.shape[0], dtype=bool)
    expect = np.zeros(bt.shape[0], dtype=np.int64)
    for first, n, P in groups:
        if not (1 <= n <= 8) or first < 0 or first + n > bt.shape[0] or P % bs or P > max_prefix_len:
            raise ValueError(f"bad prefix group {(first, n, P)}")
        if covered[first:first + n].any():
            raise ValueError("prefix groups overlap")
        covered[first:first + n] = True
        expect[first:first + n] = P
        for s in range(first, first + n):
            if lens[s] < P or (bt[s, : P // bs] != bt[first, : P // bs]).any():
                raise ValueError(f"sequence {s} does not share group {first}'s prefix")
    if (pre != expect).any():
        raise ValueError("seq_prefix_lens disagrees with prefix_groups")


def pa_prefill_chunk(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                     max_query_len: int, scale: float, check_device_args=False):
    nb, kvh, d, bs = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _arg(dev, "out", out)
    _arg(dev, "q", q)
    _arg(dev, "block_tables", block_tables, torch.int32)
    _arg(dev, "query_start_loc", query_start_loc, torch.int32)
    _arg(dev, "context_lens", context_lens, torch.int32)
    T, H = q.shape[0], q.shape[1]
    B = context_lens.shape[0]
    if q.shape != (T, H, d) or out.shape != q.shape or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q/out must be contiguous [T, H, head_dim]")
    if q.dtype != k_cache.dtype or out.dtype != q.dtype:
        raise TypeError("q/out dtype must match the cache")
    if query_start_loc.dtype != torch.int32 or query_start_loc.shape != (B + 1,):
        raise ValueError("query_start_loc must be int32 [B+1]")
    if block_tables.dtype != torch.int32 or block_tables.shape[0] != B or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, max_blocks]")
    if check_device_args:
        _check_tables(block_tables, context_lens, nb, bs)
        qsl = query_start_loc.cpu().numpy()
        lens = context_lens.cpu().numpy()
        nq = np.diff(qsl)
        if qsl[0] != 0 or qsl[-1] != T or (nq < 0).any() or (nq > max_query_len).any() or (nq > lens).any():
            raise ValueError("query_start_loc inconsistent with q / context_lens")
    check("pa_prefill_chunk", lib().pa_prefill_chunk(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.shape[1], query_start_loc.data_ptr(),
        context_lens.data_ptr(), B, int(max_query_len), H, kvh, d, bs, nb, float(scale),
        _dtype(q), _stream(q)))


def pa_mixed_step(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                  num_prefill_tokens: int, max_query_len: int, max_decode_context: int,
                  scale: float, partition: int = 0, workspace=None, check_device_args=False,
                  stream_kv: bool = False):
    """Prefill chunks (the first len(query_start_loc) - 1 sequences) and decode
    tokens (the rest, one query row each, after the chunks' rows) in one
    launch (plus the decode merge when partitioned)."""
    nb, kvh, d, bs = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _arg(dev, "out", out)
    _arg(dev, "q", q)
    _arg(dev, "block_tables", block_tables, torch.int32)
    _arg(dev, "query_start_loc", query_start_loc, torch.int32)
    _arg(dev, "context_lens", context_lens, torch.int32)
    if workspace is not None:
        _arg(dev, "workspace", workspace)
    T, H = q.shape[0], q.shape[1]
    B = context_lens.shape[0]
    P = query_start_loc.shape[0] - 1
    Dn = B - P
    if P < 0 or Dn < 0 or T != num_prefill_tokens + Dn:
        raise ValueError("q rows must be the chunks' rows followed by one row per decode sequence")
    if q.shape != (T, H, d) or out.shape != q.shape or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q/out must be contiguous [T, H, head_dim]")
    if q.dtype != k_cache.dtype or out.dtype != q.dtype:
        raise TypeError("q/out dtype must match the cache")
    if query_start_loc.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("query_start_loc and context_lens must be int32")
    if block_tables.dtype != torch.int32 or block_tables.shape[0] != B or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [B, max_blocks]")
    if check_device_args:
        _check_tables(block_tables, context_lens, nb, bs)
        qsl = query_start_loc.cpu().numpy()
        lens = context_lens.cpu().numpy()
        nq = np.diff(qsl)
        if qsl[0] != 0 or qsl[-1] != num_prefill_tokens or (nq < 0).any() \
                or (nq > max_query_len).any() or (nq > lens[:P]).any():
            raise ValueError("query_start_loc inconsistent with the chunks")
        if Dn and (lens[P:].max() > max_decode_context or lens[P:].min() < 0):
            raise ValueError("a decode context exceeds max_decode_context")
    need = int(lib().pa_mixed_step_workspace_bytes(Dn, H, d, int(max_decode_context),
                                                   int(partition)))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("pa_mixed_step", lib().pa_mixed_step(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.shape[1],
        query_start_loc.data_ptr() if P else None, context_lens.data_ptr(), P,
        int(num_prefill_tokens), int(max_query_len), Dn, int(max_decode_context), H, kvh, d, bs,
        nb, float(scale), int(partition), wptr, wbytes, _dtype(q), _flags(stream_kv), _stream(q)))
