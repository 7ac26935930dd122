"""Oracle for the paged-attention hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU implementation in float64 (numpy) of what
the paged KV-cache path computes: the block allocator, the slot mapping, the
cache write, the copy-on-write block copy, decode attention and chunked-prefill
attention over K/V gathered through a block table.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it; the two meet only in the seeded inputs of ``synth``.

Sources (web pages about vLLM's PagedAttention):
  * "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill theo
    khối & Prefix Caching" (locionic.com, Vietnamese) -- called "the deep-dive
    page" below; the only page with mechanism detail.
  * "vLLM" (tellworld.net) -- "the encyclopaedic page".
  * "vLLM PagedAttention: LLM Çıkarım Veriminde Bir Devrim" (tr.news.hada.io)
    -- "the summary page".
  * the skymod.tech article on vLLM (Turkish) -- "the overview page".

Parity pins: every function here is pinned by CPU tests against something other
than itself (a library routine, closed forms, invariants, the worked
block-table example the deep-dive page prints).  No function is "parity
unpinned".
"""
