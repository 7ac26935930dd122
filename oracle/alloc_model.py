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

Automatic prefix caching (deep-dive page, section "Cơ chế APC", items 1-2,
and its advice to evict blocks not recently used under memory pressure),
with the readings taken here:
  * a trie whose nodes are whole blocks: a node is one full block's token ids
    below the node of the blocks before it, and names the physical block that
    holds their K/V;
  * a block joins the trie when an append with token ids fills it, provided
    every earlier token id of the sequence is known and its parent path is
    still in the trie, and no node with the same token ids hangs under that
    parent already (then the sequence follows that node and its own block
    stays private); an append without token ids ends caching for the
    sequence;
  * a new request walks the trie from the root over its prompt's full
    blocks, at most (n - 1) // block_size of them (the last prompt token is
    always computed), links every matched block (one more reference) and
    starts at the matched length; hit rate = matched tokens / prompt tokens;
  * a trie block whose last reference goes away is kept, not freed; blocks
    are taken from the free list first, and only when it is empty from the
    kept ones: least recently used first (a use is a match, a registration or
    the release), deeper first among equals, then lower block id; evicting a
    block removes its node and all nodes below it, whose blocks become
    ordinary (freed, in depth-first order with children by token ids, if no
    sequence holds them).
"""

from __future__ import annotations

OK = 0
ERR_INVALID_ARG = -1
ERR_NO_FREE_BLOCKS = -2
ERR_UNKNOWN_SEQ = -3
ERR_SEQ_EXISTS = -4


class _TrieNode:
    def __init__(self, parent, depth: int, block: int):
        self.parent = parent
        self.depth = depth
        self.block = block
        self.children = {}  # tuple of token ids -> _TrieNode
        self.alive = True


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
        # prefix caching (off until enable_prefix_cache)
        self.apc = False
        self.clock = 0
        self.root = None
        self.cached = {}      # block -> _TrieNode
        self.last_use = {}    # block -> clock of its last use
        self.tokens = {}      # seq -> list of token ids, or None when unknown
        self.walk = {}        # seq -> trie node of its full blocks, or None
        self.hit_tokens = self.query_tokens = self.evictions = 0

    # --- prefix cache internals ------------------------------------------
    def _kept(self):
        """Cached blocks no sequence holds, in eviction order."""
        ks = [b for b in self.cached if self.refcount[b] == 0]
        return sorted(ks, key=lambda b: (self.last_use[b], -self.cached[b].depth, b))

    def _available(self) -> int:
        return len(self.free) + (len(self._kept()) if self.apc else 0)

    def _drop(self, node, keep):
        """Remove node and its subtree from the trie."""
        for key, child in list(node.parent.children.items()):
            if child is node:
                del node.parent.children[key]
        order = []

        def visit(x):
            order.append(x)
            for key in sorted(x.children):
                visit(x.children[key])
        visit(node)
        for x in order:
            if self.refcount[x.block] == 0 and x.block != keep:
                self.free.append(x.block)
            del self.cached[x.block]
            x.alive = False

    def _take(self) -> int:
        if self.free:
            return self.free.pop()
        b = self._kept()[0]
        self._drop(self.cached[b], keep=b)
        self.evictions += 1
        return b

    def _release(self, b: int):
        if self.apc and b in self.cached:
            self.last_use[b] = self.clock
        else:
            self.free.append(b)

    def _register(self, seq: int, first: int, last: int):
        bs = self.block_size
        toks = self.tokens[seq]
        for i in range(first, last):
            node = self.walk[seq]
            if node is None or not node.alive:
                self.walk[seq] = None
                return
            key = tuple(toks[i * bs:(i + 1) * bs])
            if key in node.children:
                self.walk[seq] = node.children[key]
                continue
            b = self.tables[seq][i]
            child = _TrieNode(node, i + 1, b)
            node.children[key] = child
            self.cached[b] = child
            self.last_use[b] = self.clock
            self.walk[seq] = child

    # --- operations -----------------------------------------------------
    def enable_prefix_cache(self) -> int:
        if self.tables:
            return ERR_INVALID_ARG
        if not self.apc:
            self.apc = True
            self.root = _TrieNode(None, 0, -1)
        return OK

    def new(self, seq: int) -> int:
        if seq in self.tables:
            return ERR_SEQ_EXISTS
        self.tables[seq] = []
        self.lens[seq] = 0
        self.tokens[seq] = []
        self.walk[seq] = self.root
        return OK

    def new_cached(self, seq: int, prompt):
        """Returns (status, cached tokens)."""
        if not self.apc:
            return ERR_INVALID_ARG, 0
        if seq in self.tables:
            return ERR_SEQ_EXISTS, 0
        self.clock += 1
        bs = self.block_size
        prompt = [int(t) for t in prompt]
        node, table = self.root, []
        for i in range(max(0, (len(prompt) - 1) // bs)):
            key = tuple(prompt[i * bs:(i + 1) * bs])
            if key not in node.children:
                break
            node = node.children[key]
            self.refcount[node.block] += 1
            self.last_use[node.block] = self.clock
            table.append(node.block)
        n_hit = len(table) * bs
        self.tables[seq] = table
        self.lens[seq] = n_hit
        self.tokens[seq] = prompt[:n_hit]
        self.walk[seq] = node
        self.hit_tokens += n_hit
        self.query_tokens += len(prompt)
        return OK, n_hit

    def append_tokens(self, seq: int, toks):
        return self.append(seq, len(toks), toks)

    def append(self, seq: int, n: int, toks=None):
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
        if grow + int(cow) > self._available():
            return ERR_NO_FREE_BLOCKS, [], []
        self.clock += 1
        pairs = []
        if cow:
            src, dst = table[-1], self._take()
            self.refcount[src] -= 1
            self.refcount[dst] = 1
            table[-1] = dst
            pairs.append((src, dst))
        for _ in range(grow):
            b = self._take()
            self.refcount[b] = 1
            table.append(b)
        slots = [table[p // bs] * bs + p % bs for p in range(L, L + n)]
        self.lens[seq] = L + n
        if self.apc:
            if toks is not None and self.tokens[seq] is not None:
                self.tokens[seq].extend(int(t) for t in toks)
                self._register(seq, L // bs, (L + n) // bs)
            else:
                self.tokens[seq] = None
                self.walk[seq] = None
        return OK, slots, pairs

    def fork(self, parent: int, child: int) -> int:
        if parent not in self.tables:
            return ERR_UNKNOWN_SEQ
        if child in self.tables:
            return ERR_SEQ_EXISTS
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        t = self.tokens.get(parent)
        self.tokens[child] = None if t is None else list(t)
        self.walk[child] = self.walk.get(parent)
        for b in self.tables[child]:
            self.refcount[b] += 1
        return OK

    def free_seq(self, seq: int) -> int:
        if seq not in self.tables:
            return ERR_UNKNOWN_SEQ
        self.clock += 1
        for b in reversed(self.tables[seq]):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self._release(b)
        del self.tables[seq]
        del self.lens[seq]
        self.tokens.pop(seq, None)
        self.walk.pop(seq, None)
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

    def prefix_cache_stats(self) -> dict:
        return {"hit_tokens": self.hit_tokens, "query_tokens": self.query_tokens,
                "cached_blocks": len(self.cached), "evictable": len(self._kept()) if self.apc else 0,
                "evictions": self.evictions}

    def prefix_cache_blocks(self):
        """({block: depth} of the trie's blocks, kept blocks in eviction order)."""
        return ({b: n.depth for b, n in sorted(self.cached.items())},
                self._kept() if self.apc else [])

    def wasted_slots(self) -> int:
        """Internal fragmentation: allocated but unused slots, per sequence."""
        return sum(len(t) * self.block_size - self.lens[s] for s, t in self.tables.items())
