"""Block pool: LIFO free list, reference counts, copy-on-write (oracle).

[K3] section 1 "Block-Arena KV Cache": the free list starts as the list of all
block ids; allocating pops from its end (so the highest id comes out first)
and freeing appends, so the block freed last is the next one handed out.
[K3] section 3 "Radix-Tree Prefix Cache": shared blocks are kept alive by
reference counts, and a request that diverges inside a shared block copies
that block before writing it.

Reading of the copy-on-write order (the pages give none): if the block is
shared (count > 1), pop a fresh block, (the caller copies the data), then drop
one reference to the old block.  A block with count 1 is written in place.

[K3] section 5 "Continuous Batching and Admission Control": a new sequence is
admitted only if free + evictable >= active_reserved + new_need.
"""
from __future__ import annotations


class PoolError(Exception):
    pass


class OutOfBlocks(PoolError):
    pass


class RefcountError(PoolError):
    pass


class Pool:
    def __init__(self, num_blocks: int):
        self.num_blocks = num_blocks
        self.free = list(range(num_blocks))
        self.refcount = {}

    def alloc(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def incref(self, b: int) -> None:
        if self.refcount.get(b, 0) < 1:
            raise RefcountError(f"incref of free block {b}")
        self.refcount[b] += 1

    def decref(self, b: int) -> None:
        rc = self.refcount.get(b, 0)
        if rc < 1:
            raise RefcountError(f"decref of free block {b}")
        if rc == 1:
            del self.refcount[b]
            self.free.append(b)
        else:
            self.refcount[b] = rc - 1

    def cow(self, b: int):
        """Returns (block to write, copied?).  A fresh block when b is shared."""
        rc = self.refcount.get(b, 0)
        if rc < 1:
            raise RefcountError(f"copy-on-write of free block {b}")
        if rc == 1:
            return b, False
        nb = self.alloc()
        self.decref(b)
        return nb, True

    @property
    def num_free(self) -> int:
        return len(self.free)


def can_admit(free: int, evictable: int, active_reserved: int, new_need: int) -> bool:
    """[K3] section 5: strict admission, so that admitted sequences can always
    finish (no memory deadlock)."""
    return free + evictable >= active_reserved + new_need
