"""Oracle: a reference model of the host block allocator.

Deep-dive page ("vLLM PagedAttention chuyên sâu ..."):
  * section "Tương tự phân trang bộ nhớ ảo": a sequence's KV cache is a list of
    fixed-size logical blocks; each maps to a physical block; the block table
    is the per-sequence array from logical to physical block index; physical
    blocks may be scattered and may be shared by several sequences; a growing
    sequence gets new physical blocks without moving the old ones;
  * the listing under "Cơ chế PagedAttention": ceil(tokens / block_size)
    blocks per sequence (30 tokens -> 2 blocks, 50 tokens -> 4 blocks);
  * section "Cơ chế APC", item 3: copy-on-write -- a sequence diverging from
    shared blocks first copies the shared block it must change.
Overview page (skymod.tech): in parallel sampling the prompt's memory is
shared by the output sequences.

Policies the pages leave open (readings):
  * free list is a LIFO stack; ``free_order[0]`` is handed out first; a block
    whose reference count drops to 0 is pushed on top;
  * ``free`` releases a sequence's blocks from its last logical block to its
    first, so its first block ends on top of the stack;
  * ``fork`` gives the child the parent's table and length, and every block
    one more reference;
  * ``append`` of n tokens to a sequence of length L: if L is not a multiple
    of block_size and the last block has more than one reference, the last
    block is copied first (pop dst, report (src, dst), src loses a reference,
    dst replaces it in the table); then ceil((L+n)/block_size) - len(table)
    blocks are popped in logical order; the n slots are
    slot(p) = table[p // block_size] * block_size + p % block_size for
    p = L .. L+n-1;
  * every call either succeeds completely or changes nothing (out of blocks,
    unknown or duplicate sequence ids, negative counts).
"""

from __future__ import annotations

OK = 0
ERR_INVALID_ARG = -1
ERR_NO_FREE_BLOCKS = -2
ERR_UNKNOWN_SEQ = -3
ERR_SEQ_EXISTS = -4


class AllocModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(reversed(order))  # top of stack = end of list
        self.refcount = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    # --- operations -----------------------------------------------------
    def new(self, seq: int) -> int:
        if seq in self.tables:
            return ERR_SEQ_EXISTS
        self.tables[seq] = []
        self.lens[seq] = 0
        return OK

    def append(self, seq: int, n: int):
        """Returns (status, slots, cow_pairs)."""
        if seq not in self.tables:
            return ERR_UNKNOWN_SEQ, [], []
        if n < 0:
            return ERR_INVALID_ARG, [], []
        if n == 0:
            return OK, [], []
        bs = self.block_size
        table = self.tables[seq]
        L = self.lens[seq]
        cow = L % bs != 0 and self.refcount[table[-1]] > 1
        grow = -(-(L + n) // bs) - len(table)
        if grow + int(cow) > len(self.free):
            return ERR_NO_FREE_BLOCKS, [], []
        pairs = []
        if cow:
            src, dst = table[-1], self.free.pop()
            self.refcount[src] -= 1
            self.refcount[dst] = 1
            table[-1] = dst
            pairs.append((src, dst))
        for _ in range(grow):
            b = self.free.pop()
            self.refcount[b] = 1
            table.append(b)
        slots = [table[p // bs] * bs + p % bs for p in range(L, L + n)]
        self.lens[seq] = L + n
        return OK, slots, pairs

    def fork(self, parent: int, child: int) -> int:
        if parent not in self.tables:
            return ERR_UNKNOWN_SEQ
        if child in self.tables:
            return ERR_SEQ_EXISTS
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1
        return OK

    def free_seq(self, seq: int) -> int:
        if seq not in self.tables:
            return ERR_UNKNOWN_SEQ
        for b in reversed(self.tables[seq]):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.tables[seq]
        del self.lens[seq]
        return OK

    # --- queries --------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def block_table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def seq_len(self, seq: int) -> int:
        return self.lens[seq]

    def padded_tables(self, seqs, max_blocks: int):
        """Block tables of ``seqs`` as rows of length max_blocks, -1 padded."""
        rows = []
        for s in seqs:
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table wider than max_blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
        return rows

    def wasted_slots(self) -> int:
        """Internal fragmentation: allocated but unused slots, per sequence."""
        return sum(len(t) * self.block_size - self.lens[s] for s, t in self.tables.items())
