"""Oracle: execute a workload script with the reference allocator and the
reference cache write, and compute the step's attention outputs.

A script (see ``synth``) is a list of allocator operations; every append's
tokens are written into the slots the allocator returns, after any
copy-on-write block copy it reports (deep-dive page "vLLM PagedAttention
chuyên sâu ...", section "Cơ chế APC", item 3).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import attention, cache
from .alloc_model import OK, AllocModel


@dataclass
class OracleState:
    model: AllocModel
    k_cache: np.ndarray
    v_cache: np.ndarray
    step_slots: list = field(default_factory=list)  # slot list per step append
    cow_pairs: list = field(default_factory=list)  # every (src, dst) reported


def apply_op(st: OracleState, script, op, write_seqs=None) -> list:
    """Run one allocator operation; returns the slots of an append.  With
    ``write_seqs`` given, only appends of those sequences write K/V (the
    allocator still sees every operation, so placement is unchanged)."""
    slots = []
    if op.kind == "new":
        rc = st.model.new(op.seq)
    elif op.kind == "fork":
        rc = st.model.fork(op.parent, op.seq)
    elif op.kind == "append":
        rc, slots, pairs = st.model.append(op.seq, op.n)
        if rc == OK:
            if pairs:
                cache.copy_blocks(st.k_cache, st.v_cache, pairs)
                st.cow_pairs.extend(pairs)
            if write_seqs is None or op.seq in write_seqs:
                k, v = script.kv(op)
                cache.reshape_and_cache(k, v, st.k_cache, st.v_cache, np.asarray(slots, np.int64))
    else:
        raise ValueError(op.kind)
    if rc != OK:
        raise RuntimeError(f"oracle allocator rejected {op}: status {rc}")
    return slots


def ancestors(script, seqs) -> set:
    """``seqs`` plus every sequence they were forked from."""
    parent = {op.seq: op.parent for op in script.ops() if op.kind == "fork"}
    out = set()
    for s in seqs:
        while s not in out:
            out.add(s)
            if s not in parent:
                break
            s = parent[s]
    return out


def build(script, include_step: bool = True, poison: int | None = None,
          only_seqs=None) -> OracleState:
    """Execute the script.  ``only_seqs`` limits the cache writes to the
    tokens those sequences (and the sequences they forked from) read."""
    s = script.spec
    write = None if only_seqs is None else ancestors(script, only_seqs)
    st = OracleState(AllocModel(script.num_blocks, s.block_size, script.free_order),
                     *cache.empty_cache(script.num_blocks, s.num_kv_heads, s.head_dim,
                                        s.block_size, s.dtype, poison))
    for op in script.setup:
        apply_op(st, script, op, write)
    if include_step:
        for op in script.step:
            st.step_slots.append(apply_op(st, script, op, write))
    return st


def batch_tables(st: OracleState, script):
    tables = np.array(st.model.padded_tables(script.batch, script.max_blocks_per_seq), np.int32)
    lens = np.array([st.model.seq_len(s) for s in script.batch], np.int32)
    return tables, lens


def step_output(st: OracleState, script, q, select=None) -> np.ndarray:
    """Float64 outputs of the batch step.  ``select`` optionally lists
    (row, head) outputs to compute (row = sequence for decode, packed query
    row for prefill)."""
    s = script.spec
    tables, lens = batch_tables(st, script)
    if s.kind == "decode":
        return attention.decode(q, st.k_cache, st.v_cache, tables, lens, s.scale, s.dtype, select)
    qsl = np.concatenate([[0], np.cumsum(script.query_lens)]).astype(np.int32)
    return attention.prefill(q, st.k_cache, st.v_cache, tables, qsl, lens, s.scale, s.dtype, select)
