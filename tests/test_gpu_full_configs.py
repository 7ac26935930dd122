"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (each workload's default partition size), over the whole
output tensor.

Both sides run the whole script: the block tables must agree bit for bit for
every sequence, the whole K/V pool bit for bit (poisoned slots included), and
every output within the stated tolerance (fp32: max abs <= 1e-5; bf16: max
abs <= 2e-2 and relative L2 <= 5e-3 over the whole tensor).  The oracle is the
plain definition; prefill uses its matrix form (attention.prefill_rows,
pinned to the row-by-row oracle).  The script's K/V draws are made once and
handed to both sides.
"""

import numpy as np
import pytest
import torch

from oracle import attention, run
from synth import config_script

from .parity import assert_close, assert_pool_equal, gpu_step, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def memoize_draws(sc):
    """Make the script hand out each append's K/V draw once (both sides use
    the same seeded arrays; drawing them twice only costs time)."""
    cache = {}
    draw = sc.kv

    def kv(op):
        key = (op.stream, op.n)
        if key not in cache:
            cache[key] = draw(op)
        return cache[key]
    sc.kv = kv
    return sc


def whole_reference(sc, st):
    s = sc.spec
    tables, lens = run.batch_tables(st, sc)
    q = sc.q(0)
    if s.kind == "decode":
        return attention.decode(q, st.k_cache, st.v_cache, tables, lens, s.scale, s.dtype)
    qsl = np.concatenate([[0], np.cumsum(sc.query_lens)]).astype(np.int32)
    return attention.prefill_rows(q, st.k_cache, st.v_cache, tables, qsl, lens, s.scale, s.dtype)


@pytest.mark.parametrize("name", ["decode_bf16", "gqa_decode_bf16", "shared_prefix_bf16",
                                  "shared_prefix_bf16:grouped", "shared_prefix_bf16:found",
                                  "chunked_prefill_bf16"])
def test_full_size_whole_tensor(name):
    say(f"full-size {name}: GPU step")
    name, _, mode = name.partition(":")
    sc = memoize_draws(config_script(name))
    # grouped: through pa_decode_shared_prefix with the planner's default groups;
    # found: through pa_decode finding the groups on the device
    w, out, bt_h, lens_h = gpu_step(sc, shared_prefix=(8, 256) if mode == "grouped" else None,
                                    find_shared=mode == "found")
    if mode == "grouped":
        assert len(w.prefix_plan[0]) == len(sc.batch) // 8
    say("  oracle build (whole script)")
    st = run.build(sc)
    tables, lens = run.batch_tables(st, sc)
    assert np.array_equal(bt_h, tables), "block tables differ from the oracle allocator"
    assert np.array_equal(lens_h, lens)
    assert_pool_equal(w, st)
    say("  oracle attention (every output)")
    ref = whole_reference(sc, st)
    mx, rel = assert_close(out, ref, sc.spec.dtype, what=name)
    say(f"  {out.numel() // sc.spec.head_dim} outputs: max abs {mx:.2e} rel L2 {rel:.2e}")
