"""ctypes binding of libpa (include/pa.h): argument marshalling only.

Every function here checks shapes and dtypes on the host, then calls the
library entry point of the same name with raw device pointers and the current
HIP stream.  Nothing is computed in Python.  If libpa.so is missing the first
call raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pa.h")

PA_OK = 0
PA_F32 = 0
PA_BF16 = 1
PA_DECODE_STREAM_KV = 1
PA_DECODE_FIND_SHARED = 2
PA_FIND_SHARED_MIN_PREFIX = 256
STATUS = {0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_NO_FREE_BLOCKS",
          -3: "PA_ERR_UNKNOWN_SEQ", -4: "PA_ERR_SEQ_EXISTS", -5: "PA_ERR_UNSUPPORTED",
          -6: "PA_ERR_WORKSPACE", -7: "PA_ERR_DEVICE"}

_lock = threading.Lock()
_lib = None

c_i32, c_i64, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "pa_status_str": (ctypes.c_char_p, [c_i32]),
    "pa_version": (c_i32, []),
    "pa_reshape_and_cache": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i32,
                                     c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pa_copy_blocks": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pa_decode_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode_workspace_bytes_flags": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i32, c_i32, c_i32,
                          c_i32, c_i32, c_f32, c_i32, c_i32, c_vp, c_sz, c_i32, c_i32, c_vp]),
    "pa_decode_no_alloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i32,
                                   c_i32, c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_i32, c_i32,
                                   c_vp]),
    "pa_prefix_plan": (c_i32, [c_vp, c_i32, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                               c_vp]),
    "pa_decode_shared_prefix_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode_shared_prefix": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i32,
                                        c_i32, c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_vp,
                                        c_i32, c_vp, c_i32, c_vp, c_sz, c_i32, c_i32, c_vp]),
    "pa_prefill_chunk": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32,
                                 c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp]),
    "pa_mixed_step": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                              c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp,
                              c_sz, c_i32, c_i32, c_vp]),
    "pa_mixed_step_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_alloc_create": (c_i32, [c_i32, c_i32, c_vp, ctypes.POINTER(c_vp)]),
    "pa_alloc_destroy": (None, [c_vp]),
    "pa_seq_new": (c_i32, [c_vp, c_i64]),
    "pa_seq_fork": (c_i32, [c_vp, c_i64, c_i64]),
    "pa_seq_append": (c_i32, [c_vp, c_i64, c_i32, c_vp, c_vp, c_vp]),
    "pa_seq_free": (c_i32, [c_vp, c_i64]),
    "pa_seq_len": (c_i32, [c_vp, c_i64, c_vp]),
    "pa_seq_block_table": (c_i32, [c_vp, c_i64, c_vp, c_i32, c_vp]),
    "pa_block_refcount": (c_i32, [c_vp, c_i32, c_vp]),
    "pa_num_free": (c_i32, [c_vp, c_vp]),
    "pa_free_list": (c_i32, [c_vp, c_vp, c_i32, c_vp]),
    "pa_batch_append": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp]),
    "pa_export_tables": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_i32, c_vp]),
    "pa_alloc_stats": (c_i32, [c_vp, c_vp]),
    "pa_alloc_enable_prefix_cache": (c_i32, [c_vp]),
    "pa_seq_new_cached": (c_i32, [c_vp, c_i64, c_vp, c_i32, c_vp]),
    "pa_seq_append_tokens": (c_i32, [c_vp, c_i64, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "pa_prefix_cache_stats": (c_i32, [c_vp, c_vp]),
    "pa_prefix_cache_blocks": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_vp]),
}


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions include/pa.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


# The ABI this binding marshals for (include/pa.h, pa_version).  Version 2
# added the `flags` argument before `stream` in pa_decode,
# pa_decode_shared_prefix and pa_mixed_step: a version-1 library called with
# these argument types takes the flags as its stream.  Version 3 added
# pa_decode_workspace_bytes_flags and the PA_DECODE_FIND_SHARED flag.
ABI_VERSION = 3


def load_library(path: str, host_only: bool = False) -> ctypes.CDLL:
    """Load a libpa build and bind the argument types of its entry points.

    pa_version (whose signature never changes) is bound and called first; a
    library of another ABI version is refused before any other symbol is
    bound.  ``host_only``: bind only the symbols the file exports (a build of
    the host allocator alone, e.g. with sanitizers)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m paged_kv_cache_219_amd.build`")
    L = ctypes.CDLL(path)
    ver = L.pa_version
    ver.restype = c_i32
    ver.argtypes = []
    v = int(ver())
    if v != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {v}; this binding marshals version "
                           f"{ABI_VERSION} -- rebuild the library")
    for name, (res, args) in _SIGS.items():
        if host_only and not hasattr(L, name):
            continue
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def lib() -> ctypes.CDLL:
    """The in-tree libpa.so (or, for host-only test builds, the library named
    by the PA_HOST_LIB environment variable), loaded once."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                alt = os.environ.get("PA_HOST_LIB")
                _lib = load_library(alt, host_only=True) if alt else load_library(LIB_PATH)
    return _lib


class PagedAttentionError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


def check(fn: str, status: int) -> int:
    if status != PA_OK:
        raise PagedAttentionError(fn, status)
    return status


def ptr(a) -> int:
    """Address of a numpy array's data (host)."""
    return a.ctypes.data if a is not None else 0


# ------------------------------------------------------------------ allocator
class BlockAllocator:
    """Host block allocator (libpa's pa_alloc_* / pa_seq_* entry points)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._L = lib()
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        h = c_vp()
        fo = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        if fo is not None and fo.shape != (self.num_blocks,):
            raise ValueError("free_order must have num_blocks entries")
        check("pa_alloc_create", self._L.pa_alloc_create(self.num_blocks, self.block_size,
                                                          ptr(fo) if fo is not None else None,
                                                          ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._L.pa_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # raw status-returning calls (for lockstep tests)
    def new(self, seq: int) -> int:
        return self._L.pa_seq_new(self._h, int(seq))

    def fork(self, parent: int, child: int) -> int:
        return self._L.pa_seq_fork(self._h, int(parent), int(child))

    def append(self, seq: int, n: int):
        """Returns (status, slots list, cow pairs list)."""
        slots = np.zeros(max(int(n), 1), np.int64)
        pair = np.zeros(2, np.int32)
        ncow = np.zeros(1, np.int32)
        rc = self._L.pa_seq_append(self._h, int(seq), int(n), ptr(slots), ptr(pair), ptr(ncow))
        if rc != PA_OK:
            return rc, [], []
        return rc, slots[:n].tolist(), [(int(pair[0]), int(pair[1]))] if ncow[0] else []

    def free(self, seq: int) -> int:
        return self._L.pa_seq_free(self._h, int(seq))

    def seq_len(self, seq: int) -> int:
        out = np.zeros(1, np.int32)
        check("pa_seq_len", self._L.pa_seq_len(self._h, int(seq), ptr(out)))
        return int(out[0])

    def block_table(self, seq: int) -> list[int]:
        n = np.zeros(1, np.int32)
        check("pa_seq_block_table", self._L.pa_seq_block_table(self._h, int(seq), None, 0, ptr(n)))
        buf = np.zeros(max(int(n[0]), 1), np.int32)
        check("pa_seq_block_table",
              self._L.pa_seq_block_table(self._h, int(seq), ptr(buf), int(n[0]), ptr(n)))
        return buf[: int(n[0])].tolist()

    def refcount(self, block: int) -> int:
        out = np.zeros(1, np.int32)
        check("pa_block_refcount", self._L.pa_block_refcount(self._h, int(block), ptr(out)))
        return int(out[0])

    def num_free(self) -> int:
        out = np.zeros(1, np.int32)
        check("pa_num_free", self._L.pa_num_free(self._h, ptr(out)))
        return int(out[0])

    def free_list(self) -> list[int]:
        n = np.zeros(1, np.int32)
        buf = np.zeros(self.num_blocks, np.int32)
        check("pa_free_list", self._L.pa_free_list(self._h, ptr(buf), self.num_blocks, ptr(n)))
        return buf[: int(n[0])].tolist()

    def stats(self) -> dict:
        out = np.zeros(5, np.int64)
        check("pa_alloc_stats", self._L.pa_alloc_stats(self._h, ptr(out)))
        return dict(zip(["free", "used", "shared", "seqs", "wasted_slots"], out.tolist()))

    def batch_append(self, seqs, n, max_blocks: int, tables_out=None, lens_out=None,
                     slots_out=None, cow_out=None):
        """Appends n[i] tokens to seqs[i]; fills (and returns) slots, CoW pairs,
        padded block tables and context lengths.  Raises on failure."""
        seqs = np.ascontiguousarray(seqs, np.int64)
        n = np.ascontiguousarray(n, np.int32)
        B = len(seqs)
        total = int(n.sum())
        slots = slots_out if slots_out is not None else np.empty(max(total, 1), np.int64)
        cow = cow_out if cow_out is not None else np.empty((max(B, 1), 2), np.int32)
        tables = tables_out if tables_out is not None else np.empty((B, max_blocks), np.int32)
        lens = lens_out if lens_out is not None else np.empty(B, np.int32)
        ncow = np.zeros(1, np.int32)
        done = np.zeros(1, np.int32)
        check("pa_batch_append",
              self._L.pa_batch_append(self._h, ptr(seqs), B, ptr(n), ptr(slots), ptr(cow),
                                      ptr(ncow), ptr(tables), int(max_blocks), ptr(lens), ptr(done)))
        return slots[:total], cow[: int(ncow[0])], tables, lens

    # prefix caching
    def enable_prefix_cache(self) -> int:
        return self._L.pa_alloc_enable_prefix_cache(self._h)

    def new_cached(self, seq: int, tokens):
        """Returns (status, cached tokens)."""
        t = np.ascontiguousarray(tokens, np.int32)
        out = np.zeros(1, np.int32)
        rc = self._L.pa_seq_new_cached(self._h, int(seq), ptr(t) if t.size else None, t.size,
                                       ptr(out))
        return rc, int(out[0]) if rc == PA_OK else 0

    def append_tokens(self, seq: int, tokens):
        """Returns (status, slots list, cow pairs list)."""
        t = np.ascontiguousarray(tokens, np.int32)
        n = t.size
        slots = np.zeros(max(n, 1), np.int64)
        pair = np.zeros(2, np.int32)
        ncow = np.zeros(1, np.int32)
        rc = self._L.pa_seq_append_tokens(self._h, int(seq), ptr(t) if n else None, n, ptr(slots),
                                          ptr(pair), ptr(ncow))
        if rc != PA_OK:
            return rc, [], []
        return rc, slots[:n].tolist(), [(int(pair[0]), int(pair[1]))] if ncow[0] else []

    def prefix_cache_stats(self) -> dict:
        out = np.zeros(5, np.int64)
        check("pa_prefix_cache_stats", self._L.pa_prefix_cache_stats(self._h, ptr(out)))
        return dict(zip(["hit_tokens", "query_tokens", "cached_blocks", "evictable", "evictions"],
                        out.tolist()))

    def prefix_cache_blocks(self):
        """({block: depth} of the blocks in the trie, kept blocks in eviction order)."""
        cap = self.num_blocks
        b = np.zeros(cap, np.int32)
        d = np.zeros(cap, np.int32)
        e = np.full(cap, -1, np.int32)
        n = np.zeros(1, np.int32)
        check("pa_prefix_cache_blocks",
              self._L.pa_prefix_cache_blocks(self._h, ptr(b), ptr(d), ptr(e), cap, ptr(n)))
        k = self.prefix_cache_stats()["evictable"]
        return dict(zip(b[: int(n[0])].tolist(), d[: int(n[0])].tolist())), e[:k].tolist()

    def export_tables(self, seqs, max_blocks: int):
        seqs = np.ascontiguousarray(seqs, np.int64)
        tables = np.empty((len(seqs), max_blocks), np.int32)
        lens = np.empty(len(seqs), np.int32)
        check("pa_export_tables", self._L.pa_export_tables(self._h, ptr(seqs), len(seqs),
                                                           ptr(tables), int(max_blocks), ptr(lens)))
        return tables, lens
