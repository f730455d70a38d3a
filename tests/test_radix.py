"""Radix-tree prefix cache: the oracle (oracle/radix.py) pinned to Kshipra part
3, section 3, and the library's pkv_radix_* checked against it on random
operation sequences (host code, no GPU)."""
import copy
import os

import numpy as np
import pytest

import paged_kv_chunked_amd as pkv
from oracle import pool as opool
from oracle import radix as oradix

B = 16


def tok(*blocks):
    """Token ids: one block of 16 per argument; argument k gives ids 1000k .. 1000k + 15."""
    return np.concatenate([np.arange(16, dtype=np.int32) + 1000 * b for b in blocks])


def request(p, cache, tokens, new_blocks):
    """A request: reuse the cached prefix (incref), allocate the rest, cache all."""
    matched = list(cache.match(tokens))
    for b in matched:
        p.incref(b)
    own = [p.alloc() for _ in range(len(tokens) // B - len(matched))]
    blocks = matched + own
    cache.insert(tokens, blocks)
    return blocks


def release(p, blocks):
    for b in blocks:
        p.decref(b)


def test_eviction_rescans_so_parents_become_leaves():
    """The pages' worked bug: with one cached chain root -> A -> B held by the
    tree alone, evict(2) must free 2 blocks; a snapshot of the leaves taken
    once frees only 1 (A becomes a leaf only after B is gone)."""
    for fixed in (True, False):
        p = opool.Pool(8)
        c = oradix.RadixCache(p)
        release(p, request(p, c, tok(1, 2), None))
        assert c.nodes == 2 and p.num_free == 6
        freed = c.evict(2) if fixed else c.evict_with_snapshot(2)
        assert freed == (2 if fixed else 1)
    assert p.num_free == 7      # the buggy run freed one block


def test_prefix_reuse_and_divergence():
    p = opool.Pool(16)
    c = oradix.RadixCache(p)
    a = request(p, c, tok(1, 2, 3), None)
    b = request(p, c, tok(1, 2, 9), None)          # shares the first two blocks
    assert a[:2] == b[:2] and a[2] != b[2]
    assert p.refcount[a[0]] == 3                   # tree + two requests
    assert list(c.match(tok(1, 2, 3, 4))) == a
    assert list(c.match(np.concatenate([tok(1), np.arange(5, dtype=np.int32)]))) == a[:1]
    assert c.nodes == 4


def test_shared_blocks_stay_alive():
    p = opool.Pool(16)
    c = oradix.RadixCache(p)
    a = request(p, c, tok(1, 2), None)              # still running
    release(p, request(p, c, tok(5), None))         # finished
    assert c.evictable() == 1
    assert c.evict(5) == 1                          # only the finished one goes
    assert c.nodes == 2 and all(p.refcount[x] == 2 for x in a)
    release(p, a)
    assert c.evictable() == 2 and c.evict(5) == 2 and c.nodes == 0


def test_least_recently_used_leaf_goes_first():
    p = opool.Pool(16)
    c = oradix.RadixCache(p)
    release(p, request(p, c, tok(1, 2), None))
    release(p, request(p, c, tok(3, 4), None))
    c.match(tok(1, 2))                              # touch the first branch
    assert c.evict(1) == 1
    assert len(c.match(tok(3, 4))) == 1             # the other branch lost its leaf
    assert len(c.match(tok(1, 2))) == 2


def test_evictable_equals_what_eviction_frees():
    rng = np.random.default_rng(5)
    for _ in range(100):
        p = opool.Pool(64)
        c = oradix.RadixCache(p)
        live = []
        for _ in range(12):
            n = int(rng.integers(1, 5))
            blocks = [int(x) for x in rng.integers(0, 4, size=n)]
            live.append(request(p, c, tok(*np.cumsum(blocks) + np.arange(n) * 7), None))
            if rng.random() < 0.6:
                release(p, live.pop(int(rng.integers(len(live)))))
        c2 = copy.deepcopy(c)
        assert c.evictable() == c2.evict(10 ** 6)


# ---- the library against the oracle ------------------------------------------

@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        pytest.skip("libpkv.so not built")
    return pkv.lib()


def test_library_matches_oracle_on_random_operations(lib):
    rng = np.random.default_rng(9)
    for trial in range(30):
        N = int(rng.integers(16, 80))
        op_, lp = opool.Pool(N), pkv.Pool(N)
        oc, lc = oradix.RadixCache(op_), pkv.Radix(lp)
        olive, llive = [], []
        for step in range(60):
            r = rng.random()
            if r < 0.5:
                n = int(rng.integers(1, 6))
                keys = np.cumsum(rng.integers(0, 3, size=n)) + np.arange(n) * 11
                tokens = tok(*keys)
                if rng.random() < 0.3:                       # a partial last block
                    tokens = np.concatenate([tokens, np.arange(5, dtype=np.int32)])
                mo, ml = oc.match(tokens), lc.match(tokens)   # touch both trees alike
                assert list(mo) == [int(x) for x in ml]
                need = len(tokens) // B - len(mo)
                if need > op_.num_free:
                    short = need - op_.num_free
                    assert oc.evict(short) == lc.evict(short)
                    assert oc.nodes == lc.num_nodes
                    if need > op_.num_free:
                        continue
                ob = request(op_, oc, tokens, None)
                lb = request(lp, lc, tokens, None)
                assert list(ob) == [int(x) for x in lb]
                olive.append(ob)
                llive.append(lb)
            elif r < 0.8 and olive:
                i = int(rng.integers(len(olive)))
                release(op_, olive.pop(i))
                release(lp, llive.pop(i))
            else:
                t = int(rng.integers(0, 4))
                assert oc.evict(t) == lc.evict(t)
            assert oc.nodes == lc.num_nodes
            assert oc.evictable() == lc.evictable()
            assert op_.free == list(lp.free_list())
        del lc


def test_library_radix_errors(lib):
    p = pkv.Pool(4)
    c = pkv.Radix(p)
    with pytest.raises(pkv.PkvError):
        c.insert(tok(1), [3])                       # block 3 is free: no reference to share
    b = p.alloc()
    with pytest.raises(pkv.PkvError):
        c.insert(tok(1, 2), [b, 7])                 # out of range, nothing inserted
    assert c.num_nodes == 0 and p.refcount(b) == 1
    c.insert(tok(1), [b])
    assert c.num_nodes == 1 and p.refcount(b) == 2
    assert lib.pkv_radix_evict(None, 1) == -1
    assert lib.pkv_radix_match(c._h, None, 16, None, 0) == -1
