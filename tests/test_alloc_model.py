"""Pins of the reference allocator model (CPU only).

Besides the worked example (test_oracle_pins), the model is checked by brute
force on random operation sequences against what block sharing must mean:

* reference counts equal the number of table entries naming each block;
  a block is free exactly when its count is 0; free and used blocks partition
  the pool;
* a content simulation: every slot of a tiny "memory" holds the id of the
  token written there; copy-on-write pairs are applied as block copies before
  the write; after every operation each live sequence must read back, through
  its own block table, exactly the tokens it appended or inherited -- so a
  missing or misplaced copy-on-write, a wrong slot or a block handed out twice
  shows up as a sequence whose history changed under it;
* failed calls change nothing.
"""

import numpy as np
import pytest

from oracle.alloc_model import (ERR_INVALID_ARG, ERR_NO_FREE_BLOCKS, ERR_SEQ_EXISTS,
                                ERR_UNKNOWN_SEQ, OK, AllocModel)


def check_invariants(m: AllocModel):
    counts = [0] * m.num_blocks
    for t in m.tables.values():
        for b in t:
            counts[b] += 1
    assert counts == m.refcount
    free = set(m.free)
    assert len(free) == len(m.free), "a block is on the free list twice"
    for b in range(m.num_blocks):
        assert (b in free) == (m.refcount[b] == 0)
    for s, t in m.tables.items():
        assert len(t) == -(-m.lens[s] // m.block_size)


def snapshot(m: AllocModel):
    return (list(m.free), list(m.refcount), {s: list(t) for s, t in m.tables.items()}, dict(m.lens))


def random_ops(m: AllocModel, g: np.random.Generator, steps: int, memory: dict, content: dict):
    next_tok = [1]
    next_seq = [0]
    for _ in range(steps):
        live = list(m.tables)
        r = g.random()
        before = snapshot(m)
        if r < 0.15 or not live:
            s = next_seq[0]
            next_seq[0] += 1
            assert m.new(s) == OK
            content[s] = []
        elif r < 0.65:
            s = live[g.integers(len(live))]
            n = int(g.integers(0, 2 * m.block_size + 3))
            rc, slots, pairs = m.append(s, n)
            if rc == ERR_NO_FREE_BLOCKS:
                assert snapshot(m) == before and slots == [] and pairs == []
            else:
                assert rc == OK and len(slots) == n and len(pairs) <= 1
                for src, dst in pairs:
                    for o in range(m.block_size):
                        memory[dst * m.block_size + o] = memory.get(src * m.block_size + o)
                assert len(set(slots)) == n
                for sl in slots:
                    memory[sl] = next_tok[0]
                    content[s].append(next_tok[0])
                    next_tok[0] += 1
        elif r < 0.8:
            p = live[g.integers(len(live))]
            c = next_seq[0]
            next_seq[0] += 1
            assert m.fork(p, c) == OK
            content[c] = list(content[p])
        else:
            s = live[g.integers(len(live))]
            assert m.free_seq(s) == OK
            del content[s]
        check_invariants(m)
        bs = m.block_size
        for s, toks in content.items():
            t = m.tables[s]
            got = [memory.get(t[p // bs] * bs + p % bs) for p in range(m.lens[s])]
            assert got == toks, f"sequence {s} lost its history"


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("num_blocks,block_size", [(12, 4), (40, 16), (7, 1)])
def test_random_operations_keep_sharing_semantics(seed, num_blocks, block_size):
    g = np.random.default_rng(seed)
    m = AllocModel(num_blocks, block_size, g.permutation(num_blocks))
    random_ops(m, g, 300, {}, {})


def test_cow_only_when_writing_into_a_shared_partial_block():
    m = AllocModel(16, 4)
    m.new(0)
    assert m.append(0, 8)[0] == OK  # two full blocks
    m.fork(0, 1)
    rc, slots, pairs = m.append(1, 1)  # full shared tail -> new block, no copy
    assert rc == OK and pairs == []
    m.new(2)
    m.append(2, 6)  # one full + one half block
    m.fork(2, 3)
    m.fork(2, 4)
    tail = m.block_table(2)[-1]
    assert m.refcount[tail] == 3
    rc, slots, pairs = m.append(3, 1)
    assert rc == OK and len(pairs) == 1 and pairs[0][0] == tail
    assert m.refcount[tail] == 2 and m.block_table(3)[-1] == pairs[0][1]
    assert slots == [pairs[0][1] * 4 + 2]
    rc, _, pairs = m.append(4, 3)
    assert len(pairs) == 1 and m.refcount[tail] == 1
    rc, _, pairs = m.append(2, 1)  # the last holder writes in place
    assert pairs == [] and m.block_table(2)[-1] == tail


def test_lifo_free_list_and_release_order():
    m = AllocModel(8, 2, [5, 1, 7, 0, 2, 3, 4, 6])
    m.new(0)
    _, slots, _ = m.append(0, 5)
    assert m.block_table(0) == [5, 1, 7]
    assert slots == [10, 11, 2, 3, 14]
    m.free_seq(0)
    assert m.free[-3:] == [7, 1, 5]  # first logical block on top
    m.new(1)
    m.append(1, 5)
    assert m.block_table(1) == [5, 1, 7]


def test_errors_change_nothing():
    m = AllocModel(4, 4)
    assert m.new(0) == OK
    assert m.new(0) == ERR_SEQ_EXISTS
    assert m.append(9, 1)[0] == ERR_UNKNOWN_SEQ
    assert m.append(0, -1)[0] == ERR_INVALID_ARG
    assert m.fork(9, 1) == ERR_UNKNOWN_SEQ
    assert m.fork(0, 0) == ERR_SEQ_EXISTS
    assert m.free_seq(9) == ERR_UNKNOWN_SEQ
    before = snapshot(m)
    assert m.append(0, 17)[0] == ERR_NO_FREE_BLOCKS
    assert snapshot(m) == before
    assert m.append(0, 16)[0] == OK and m.num_free() == 0
    m.fork(0, 1)
    m.free_seq(0)
    assert m.num_free() == 0
    m.free_seq(1)
    assert m.num_free() == 4


def test_cow_out_of_blocks_is_atomic():
    m = AllocModel(2, 4)
    m.new(0)
    m.append(0, 3)
    m.fork(0, 1)
    m.new(2)
    m.append(2, 1)  # pool now empty
    before = snapshot(m)
    assert m.append(1, 1)[0] == ERR_NO_FREE_BLOCKS  # needs a copy-on-write block
    assert snapshot(m) == before


def test_wasted_slots_below_block_size_per_sequence():
    g = np.random.default_rng(3)
    m = AllocModel(400, 16, g.permutation(400))
    for s in range(20):
        m.new(s)
        m.append(s, int(g.integers(1, 300)))
        assert 0 <= m.wasted_slots() < 16 * (s + 1)
