"""Model block allocator: free pool, refcounts, copy-on-write, sequence growth.

TEST INFRASTRUCTURE (see the package docstring): the native allocator must
match this model bit for bit on every operation trace.

The steps follow the explainer ["PagedAttention Nedir?", section
"PagedAttention Nasıl Çalışır?"]: (1) K/V live in fixed-size blocks, (2) a
sequence takes blocks as it grows, (3) a block table records where each
logical block lives, (5) blocks no longer needed are reused. The
PagedAttention newsletter ["İddia ve Gerçeklik"] adds: a free block is taken
from the pool when the current block is full, and parallel samples share
blocks by reference with copy-on-write.

Policy readings (the pages allow any free block; one rule is fixed so both
implementations agree exactly):
  * the free pool is a FIFO queue; it starts in ``free_order`` (or 0..N-1);
    allocation pops from the head; a block whose refcount reaches zero is
    appended at the tail, in the order the caller listed it;
  * allocate -> refcount 1; share -> +1; free -> -1; any operation on a block
    with refcount 0 is an error (EREFCOUNT);
  * copy-on-write of a block with refcount 1 keeps it; with refcount > 1 it
    takes a new block (refcount 1), drops one reference to the old one, and
    reports that the contents must be copied;
  * a sequence appending the token at position p takes a new block when
    p % B == 0, otherwise it writes into the block holding p, after
    copy-on-write if that block is shared;
  * every operation is all-or-nothing: on error nothing changes.
"""
from __future__ import annotations

from collections import deque

from . import attention as _att

OK = 0
EINVAL = -1
ENOMEM = -2
EREFCOUNT = -3


class ModelPool:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("bad pool shape")
        order = list(range(num_blocks)) if free_order is None else [
            int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..N-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.rc = [0] * num_blocks

    # -- snapshots make every composite operation all-or-nothing ----------
    def _snapshot(self):
        return deque(self.free), list(self.rc)

    def _restore(self, snap):
        self.free, self.rc = snap

    def _valid(self, b) -> bool:
        return 0 <= int(b) < self.num_blocks

    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, b: int) -> int:
        return self.rc[b] if self._valid(b) else EINVAL

    def alloc(self, n: int):
        """Take n blocks from the head of the free queue -> (status, ids)."""
        if n < 0:
            return EINVAL, []
        if n > len(self.free):
            return ENOMEM, []
        ids = [self.free.popleft() for _ in range(n)]
        for b in ids:
            self.rc[b] = 1
        return OK, ids

    def free_blocks(self, ids) -> int:
        """Drop one reference per listed id (an id may repeat)."""
        if any(not self._valid(b) for b in ids):
            return EINVAL
        need = {}
        for b in ids:
            need[int(b)] = need.get(int(b), 0) + 1
        if any(self.rc[b] < c for b, c in need.items()):
            return EREFCOUNT
        for b in ids:
            b = int(b)
            self.rc[b] -= 1
            if self.rc[b] == 0:
                self.free.append(b)
        return OK

    def share(self, ids) -> int:
        """Add one reference per listed id (fork of a sequence)."""
        if any(not self._valid(b) for b in ids):
            return EINVAL
        if any(self.rc[int(b)] == 0 for b in ids):
            return EREFCOUNT
        for b in ids:
            self.rc[int(b)] += 1
        return OK

    def cow(self, b: int):
        """-> (status, block to write into, need_copy)."""
        if not self._valid(b):
            return EINVAL, -1, 0
        if self.rc[b] == 0:
            return EREFCOUNT, -1, 0
        if self.rc[b] == 1:
            return OK, b, 0
        if not self.free:
            return ENOMEM, -1, 0
        new = self.free.popleft()
        self.rc[new] = 1
        self.rc[b] -= 1
        return OK, new, 1


def append_tokens(pool: ModelPool, tables, lens, n_new, table_capacity: int):
    """Grow sequences in ascending order; sequence s gains n_new[s] tokens.

    tables: list of per-sequence lists of physical ids (modified in place).
    lens: list of current lengths (modified in place).
    Returns (status, slots, cow_pairs): one slot per new token, in sequence
    order then position order, and the (src, dst) block copies the
    copy-on-writes require. On error nothing changes.
    """
    snap = pool._snapshot()
    saved_tables = [list(t) for t in tables]
    saved_lens = list(lens)
    B = pool.block_size
    slots, pairs = [], []

    def fail(st):
        pool._restore(snap)
        for s in range(len(tables)):
            tables[s][:] = saved_tables[s]
        lens[:] = saved_lens
        return st, [], []

    for s in range(len(lens)):
        if n_new[s] < 0 or lens[s] < 0:
            return fail(EINVAL)
        for _ in range(int(n_new[s])):
            p = lens[s]
            lb, off = divmod(p, B)
            if lb >= table_capacity:
                return fail(EINVAL)
            if off == 0:
                st, ids = pool.alloc(1)
                if st != OK:
                    return fail(st)
                tables[s].append(ids[0])
            else:
                st, blk, need = pool.cow(tables[s][lb])
                if st != OK:
                    return fail(st)
                if need:
                    pairs.append((tables[s][lb], blk))
                    tables[s][lb] = blk
            slots.append(_att.slot_of(tables[s], p, B))
            lens[s] = p + 1
    return OK, slots, pairs


def release_sequence(pool: ModelPool, table) -> int:
    """Step 5: a finished sequence drops its reference to every block."""
    return pool.free_blocks(list(table))
