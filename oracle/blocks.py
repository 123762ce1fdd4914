"""Block bookkeeping of the paged cache, as plain Python lists.

Test infrastructure: the reference model the library's host block manager is
checked against.

"spark_runtime/kv_cache.rs", ``PagedKvCache``: ``free_blocks`` and
``block_ref_counts`` (one count per block, so that blocks can be shared, e.g.
by a common prefix; a block handed out counts 1 and goes back to the free
list when its count reaches 0).  "combs_models/kv.rs": ``PageAllocator`` (a
stack of free page ids, filled in reverse so that page 0 comes out first),
``ensure_pages`` (append pages until the table covers the length; running
out is an error), ``popn`` (drop the last n tokens, at most the length, and
free the trailing pages that are no longer used; returns the count),
``reset`` and ``pages_used``.

Readings (the pages leave these open):
  * Sequence ids are the lowest id not in use.
  * A fork shares every block of its parent (counts go up) and copies the
    length.
  * Appending into a partly filled last block that another sequence also
    holds first moves the sequence to a fresh block (copy on write); the
    caller copies the old block's bytes into it.  The fresh block is taken
    before any new block, and the old block's count drops by one.
  * Released blocks go back on the stack last block first (popn, free).
  * A call that fails changes nothing; running out of blocks is its own
    error.
"""
from __future__ import annotations


class Exhausted(Exception):
    pass


class Blocks:
    def __init__(self, num_blocks: int, block_size: int):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.reset()

    def reset(self):
        self.free = list(range(self.num_blocks - 1, -1, -1))   # page 0 on top
        self.count = [0] * self.num_blocks
        self.seqs = {}                                          # id -> [len, table]

    # -- the allocator
    def _take(self) -> int:
        b = self.free.pop()
        self.count[b] = 1
        return b

    def _release(self, b: int):
        self.count[b] -= 1
        if self.count[b] == 0:
            self.free.append(b)

    def _pages(self, length: int) -> int:
        return -(-length // self.block_size)

    def _new_id(self) -> int:
        i = 0
        while i in self.seqs:
            i += 1
        return i

    # -- sequences
    def seq_new(self) -> int:
        i = self._new_id()
        self.seqs[i] = [0, []]
        return i

    def seq_fork(self, parent: int) -> int:
        length, table = self.seqs[parent]
        i = self._new_id()
        for b in table:
            self.count[b] += 1
        self.seqs[i] = [length, list(table)]
        return i

    def seq_free(self, s: int):
        _, table = self.seqs.pop(s)
        for b in reversed(table):
            self._release(b)

    def append(self, s: int, n: int):
        """Slots of the n new positions and the copy-on-write pair (or (-1, -1))."""
        length, table = self.seqs[s]
        bs = self.block_size
        cow = n > 0 and length % bs != 0 and self.count[table[-1]] > 1
        grow = self._pages(length + n) - len(table)
        if grow + int(cow) > len(self.free):
            raise Exhausted()
        pair = (-1, -1)
        if cow:
            old = table[-1]
            table[-1] = self._take()
            self._release(old)
            pair = (old, table[-1])
        for _ in range(grow):
            table.append(self._take())
        slots = [table[p // bs] * bs + p % bs for p in range(length, length + n)]
        self.seqs[s][0] = length + n
        return slots, pair

    def append_many(self, seqs, counts):
        """Several appends in list order after one check of the free blocks
        against the sum of every sequence's own need (its new pages, plus
        one for a shared, partly filled last page)."""
        if len(set(seqs)) != len(seqs):
            raise ValueError("repeated sequence")
        need = 0
        for s, n in zip(seqs, counts):
            length, table = self.seqs[s]
            shared = n > 0 and length % self.block_size != 0 and self.count[table[-1]] > 1
            need += self._pages(length + n) - len(table) + int(shared)
        if need > len(self.free):
            raise Exhausted()
        slots, pairs = [], []
        for s, n in zip(seqs, counts):
            sl, pair = self.append(s, n)
            slots += sl
            pairs.append(pair)
        return slots, pairs

    def popn(self, s: int, n: int) -> int:
        length, table = self.seqs[s]
        k = min(n, length)
        self.seqs[s][0] = length - k
        keep = self._pages(length - k)
        while len(table) > keep:
            self._release(table.pop())
        return k

    def table(self, seqs, max_blocks: int):
        rows, lens = [], []
        for s in seqs:
            length, t = self.seqs[s]
            if len(t) > max_blocks:
                raise ValueError("more blocks than the table holds")
            rows.append(list(t) + [-1] * (max_blocks - len(t)))
            lens.append(length)
        return rows, lens
