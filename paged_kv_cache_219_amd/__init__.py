"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libpa.so`` (C ABI in ``include/pa.h``): a host block
allocator plus HIP kernels for the cache write, copy-on-write block copies,
decode attention with split-context partitions, and chunked prefill on
matrix cores.  This package is a thin binding over it; importing it does not
load the library -- the first call does, and fails loudly if it is not built.
"""

from ._lib import BlockAllocator, PagedAttentionError, header_functions, lib  # noqa: F401

__all__ = ["BlockAllocator", "PagedAttentionError", "header_functions", "lib"]
