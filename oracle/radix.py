"""Radix-tree prefix cache over arena blocks (oracle; test infrastructure only).

[K3] section 3 "Radix-Tree Prefix Cache and the Eviction Bug": KV blocks live
in a radix tree keyed by token blocks; a new request walks the tree, reuses
every matching block and computes only the rest; reference counts keep shared
blocks alive; under memory pressure the cache evicts the least recently used
leaf.  The pages' bug listed the leaves once and looped over that list, so a
parent that became a leaf was never considered (evict(2) freed 1 block); the
fix re-scans the tree for the least recently used leaf on every iteration and
stops when nothing is evictable.

Readings (the pages leave these open):
  * a node is one full block of 16 token ids (partial blocks are not cached)
    and holds one physical block id; the tree owns one reference to it in
    the block pool;
  * match returns the blocks of the longest cached prefix of whole blocks and
    marks them used now; it takes no reference (a request adopting them
    increfs each one);
  * insert adds the blocks of a sequence's whole-block prefix that are not in
    the tree yet (existing nodes keep their block);
  * a leaf is evictable when the tree holds the only reference to its block;
    "least recently used" orders by the last match or insert that touched the
    node, ties broken by the lower node creation number;
  * evictable() counts the blocks repeated eviction could free: nodes whose
    block is referenced by the tree alone and whose whole subtree is evictable
    (the "evictable" of the admission rule, section 5).
"""
from __future__ import annotations

BLOCK = 16


class Node:
    __slots__ = ("key", "block", "parent", "children", "last", "serial")

    def __init__(self, key, block, parent, serial):
        self.key = key
        self.block = block
        self.parent = parent
        self.children = {}
        self.last = 0
        self.serial = serial


class RadixCache:
    def __init__(self, pool):
        self.pool = pool
        self.root = Node(None, -1, None, -1)
        self.clock = 0
        self.serial = 0
        self.nodes = 0

    def _keys(self, tokens):
        n = len(tokens) // BLOCK
        return [tuple(int(t) for t in tokens[i * BLOCK:(i + 1) * BLOCK]) for i in range(n)]

    def match(self, tokens):
        self.clock += 1
        node, out = self.root, []
        for key in self._keys(tokens):
            child = node.children.get(key)
            if child is None:
                break
            child.last = self.clock
            out.append(child.block)
            node = child
        return out

    def insert(self, tokens, blocks):
        self.clock += 1
        node = self.root
        for key, b in zip(self._keys(tokens), blocks):
            child = node.children.get(key)
            if child is None:
                child = Node(key, int(b), node, self.serial)
                self.serial += 1
                self.nodes += 1
                self.pool.incref(int(b))
                node.children[key] = child
            child.last = self.clock
            node = child

    def _all(self):
        stack = list(self.root.children.values())
        while stack:
            n = stack.pop()
            yield n
            stack.extend(n.children.values())

    def lru_leaf(self):
        """Re-scans the whole tree (the pages' fix)."""
        best = None
        for n in self._all():
            if n.children or self.pool.refcount.get(n.block, 0) != 1:
                continue
            if best is None or (n.last, n.serial) < (best.last, best.serial):
                best = n
        return best

    def evict(self, target: int) -> int:
        freed = 0
        while freed < target:
            leaf = self.lru_leaf()
            if leaf is None:
                break                       # nothing evictable left
            del leaf.parent.children[leaf.key]
            self.nodes -= 1
            self.pool.decref(leaf.block)
            freed += 1
        return freed

    def evict_with_snapshot(self, target: int) -> int:
        """The pages' bug, kept for the test that shows it: the evictable leaves
        are listed once, in LRU order, and only that list is walked."""
        leaves = sorted((n for n in self._all()
                         if not n.children and self.pool.refcount.get(n.block, 0) == 1),
                        key=lambda n: (n.last, n.serial))
        freed = 0
        for leaf in leaves:
            if freed >= target:
                break
            del leaf.parent.children[leaf.key]
            self.nodes -= 1
            self.pool.decref(leaf.block)
            freed += 1
        return freed

    def evictable(self) -> int:
        def walk(n):
            count, whole = 0, True
            for c in n.children.values():
                cc, cw = walk(c)
                count += cc
                whole = whole and cw
            if n is self.root:
                return count, whole
            if whole and self.pool.refcount.get(n.block, 0) == 1:
                return count + 1, True
            return count, False
        return walk(self.root)[0]
