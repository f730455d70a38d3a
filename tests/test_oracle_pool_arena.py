"""Pins for oracle.pool and oracle.arena (CPU only).

  * the LIFO free list against the worked example in tests/golden/lifo_pool.txt
    (Kshipra part 3, section 1: pop() returns the highest id first, a freed
    block is the next one handed out);
  * reference counts and copy-on-write rules (part 3, section 3), and
    conservation of blocks over random operation sequences;
  * KV sizing against the figures the pages print (tests/golden/kv_sizing.txt);
  * arena slot placement against a brute-force per-element loop.
"""
import os

import numpy as np
import pytest

from oracle import arena, pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_lifo_worked_example():
    p = pool.Pool(8)
    for line in open(os.path.join(GOLDEN, "lifo_pool.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        op, arg = line[0], int(line[1])
        if op == "alloc":
            assert p.alloc() == arg
        elif op == "free":
            p.decref(arg)
        elif op == "free_count":
            assert p.num_free == arg


def test_fresh_pool_pops_highest_first():
    p = pool.Pool(32)
    assert [p.alloc() for _ in range(5)] == [31, 30, 29, 28, 27]


def test_out_of_blocks():
    p = pool.Pool(2)
    p.alloc(), p.alloc()
    with pytest.raises(pool.OutOfBlocks):
        p.alloc()


def test_refcount_and_cow():
    p = pool.Pool(4)
    b = p.alloc()                      # 3
    p.incref(b)                        # shared by two owners
    nb, copied = p.cow(b)
    assert copied and nb == 2 and p.refcount[b] == 1 and p.refcount[nb] == 1
    same, copied = p.cow(b)            # sole owner now: written in place
    assert not copied and same == b
    p.decref(b)
    assert p.alloc() == b              # freed block reused next
    with pytest.raises(pool.RefcountError):
        p.decref(1)                    # never allocated
    with pytest.raises(pool.RefcountError):
        p.incref(0)


def test_random_ops_conserve_blocks():
    rng = np.random.default_rng(0)
    p = pool.Pool(50)
    held = []                          # one entry per reference
    for _ in range(5000):
        r = rng.random()
        if r < 0.4 and p.num_free:
            held.append(p.alloc())
        elif r < 0.55 and held:
            b = held[rng.integers(len(held))]
            p.incref(b)
            held.append(b)
        elif r < 0.7 and held:
            i = rng.integers(len(held))
            nb, copied = p.cow(held[i]) if p.num_free or held.count(held[i]) == 1 else (held[i], False)
            held[i] = nb
        elif held:
            i = rng.integers(len(held))
            p.decref(held.pop(i))
        live = set(held)
        assert p.num_free + len(live) == 50
        for b in live:
            assert p.refcount[b] == held.count(b)
        assert len(set(p.free)) == len(p.free) and not (set(p.free) & live)


def test_kv_sizing_golden():
    for line in open(os.path.join(GOLDEN, "kv_sizing.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        layers, hkv, d, nbytes, tokens, expected = map(int, line)
        per_layer = arena.Arena(1, hkv, d, np.float16 if nbytes == 2 else np.float32)
        block_bytes = per_layer.k[0].nbytes + per_layer.v[0].nbytes   # one 16-token block
        assert layers * tokens * block_bytes // arena.BLOCK == expected


def test_arena_slots_brute_force():
    rng = np.random.default_rng(2)
    N, H, D = 12, 3, 32
    a = arena.Arena(N, H, D, np.float16)
    table = rng.permutation(N)[:5]
    start, n = 7, 60
    k = rng.standard_normal((n, H, D)).astype(np.float16)
    v = rng.standard_normal((n, H, D)).astype(np.float16)
    a.write(table, start, k, v)
    x = 8                                   # fp16: 8 elements per 16-byte piece
    exp_k = np.full((N, H, D // x, 16, x), np.nan, np.float16)
    exp_v = np.full((N, H, D, 16), np.nan, np.float16)
    for t in range(n):
        pos = start + t
        blk, slot = table[pos // 16], pos % 16
        for h in range(H):
            for d in range(D):
                exp_k[blk, h, d // x, slot, d % x] = k[t, h, d]
                exp_v[blk, h, d, slot] = v[t, h, d]
    assert np.array_equal(a.k.view(np.uint16), exp_k.view(np.uint16))
    assert np.array_equal(a.v.view(np.uint16), exp_v.view(np.uint16))
    K, V = a.gather(table, start + n)
    assert np.array_equal(K[start:], k) and np.array_equal(V[start:], v)
    assert np.isnan(K[:start].astype(np.float32)).all()


def test_symbolic_arena_tracks_copies():
    s = arena.SymbolicArena(6)
    s.write([5, 4], 0, 20, source=3)
    s.copy_block(4, 1)
    src, tok = s.provenance([5, 1], 20)
    assert (src == 3).all() and (tok == np.arange(20)).all()


# ---- [K3] section 5: preemption by swapping, admission control -------------

def test_swap_roundtrip_relocates_sequence():
    """A sequence swapped out and restored into other blocks reads back the
    same K/V through its new block table (the arena layout is unchanged)."""
    rng = np.random.default_rng(7)
    a = arena.Arena(12, 2, 16, np.float16)
    a.k[:] = rng.standard_normal(a.k.shape).astype(np.float16)
    a.v[:] = rng.standard_normal(a.v.shape).astype(np.float16)
    old, new, L = [5, 2, 9], [1, 11, 0], 40
    packed = a.swap_out(old)
    b = arena.Arena(12, 2, 16, np.float16)          # all NaN
    b.swap_in(new, packed)
    k0, v0 = a.gather(old, L)
    k1, v1 = b.gather(new, L)
    assert np.array_equal(k0.view(np.uint16), k1.view(np.uint16))
    assert np.array_equal(v0.view(np.uint16), v1.view(np.uint16))
    # blocks not named are untouched (still NaN)
    assert np.isnan(b.k[3]).all() and np.isnan(b.v[3]).all()


@pytest.mark.parametrize("dtype,esize", [(np.float16, 2), (np.float32, 4)])
def test_swap_size_is_kv_bytes_per_token(dtype, esize):
    """[K3] section 1: KV bytes per token and layer = 2 x KV heads x head dim x
    bytes per element; a swapped block carries 16 tokens of it."""
    H, D, n = 8, 128, 3
    a = arena.Arena(4, H, D, dtype)
    a.k[:] = 0
    a.v[:] = 0
    assert a.swap_out([0, 3, 1]).size == n * 16 * (2 * H * D * esize)


def test_admission_rule_prevents_deadlock():
    """[K3] section 5: admitting only when free + evictable >= active_reserved +
    new_need means the admitted sequences can always be driven to completion:
    in random interleavings of block allocations no allocation ever fails."""
    rng = np.random.default_rng(3)
    for trial in range(200):
        N = int(rng.integers(8, 40))
        p = pool.Pool(N)
        active = {}          # seq -> blocks still to allocate
        held = {}
        seq = 0
        for _ in range(200):
            if rng.random() < 0.4:
                need = int(rng.integers(1, N // 2 + 1))
                reserved = sum(active.values())
                if pool.can_admit(p.num_free, 0, reserved, need):
                    active[seq], held[seq] = need, []
                    seq += 1
            elif active:
                s = int(rng.choice(list(active)))
                held[s].append(p.alloc())        # must never raise
                active[s] -= 1
                if active[s] == 0:               # finished: free everything
                    for b in held.pop(s):
                        p.decref(b)
                    del active[s]
    # and the rule is tight: without it the same demand can run out of blocks
    p = pool.Pool(4)
    with pytest.raises(pool.OutOfBlocks):
        for _ in range(5):
            p.alloc()


def test_admission_boundary():
    assert pool.can_admit(3, 1, 2, 2)        # equality admits
    assert not pool.can_admit(3, 1, 2, 3)
    assert pool.can_admit(0, 5, 0, 5)        # evictable blocks count
