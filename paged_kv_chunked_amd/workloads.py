"""Seeded synthetic inputs for paged-KV attention (shared by tests, bench and smoke).

This module only draws random numbers and describes *what happens* to a block
pool; it computes nothing the method computes (no RoPE, no attention, no block
table).  Both the HIP library's harness and the CPU oracle execute the same
pool script on their own pool implementation and append the same raw K/V.

A workload is:
  * geometry: query/KV heads, head dim, block size 16, storage dtype, RoPE theta;
  * an arena of ``num_blocks`` fixed-size blocks (Kshipra page 3, section 1:
    KV memory reserved once as fixed-size blocks handed out by a LIFO free list);
  * a pool script, an ordered list of operations:
      ("shuffle", perm)            pop every block, then free them in ``perm`` order
                                   (so later allocations come out in reverse
                                   ``perm`` order: a fully shuffled LIFO list)
      ("alloc", seq_ids)           one block for each entry of ``seq_ids``, in order,
                                   appended to that sequence's block table
      ("fill", i, seq, start, n)   append ``n`` tokens of raw K/V (fill ``i``) to
                                   ``seq`` at absolute positions start..start+n-1
      ("fork", child, parent)      child's table := parent's table, sharing blocks
                                   (Kshipra page 3, section 3: refcounted prefix)
      ("cow", seq, logical)        copy-on-write of ``seq``'s logical block
      ("release", seq)             drop every block reference held by ``seq``
  * a step: the batch the hot path runs on, a list of (seq, start P, count C).
    C == 1 is a decode token at position P (context length P + 1); C > 1 is a
    prefill chunk at positions P..P+C-1 (Kshipra page 3, section 4).

Random draws: ``numpy.random.default_rng(SeedSequence(seed, spawn_key=...))``
per fill and per step sequence, float32 N(0, 1) then cast to the storage dtype
with numpy round-to-nearest-even.  Per-fill streams let a test regenerate a
subset of sequences without drawing the whole workload.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import List, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16

_DTYPES = {"f16": np.float16, "f32": np.float32}


@dataclasses.dataclass(frozen=True)
class StepSeq:
    seq: int     # pool sequence id whose block table this row uses
    start: int   # absolute position P of the first new token
    count: int   # number of new tokens C (1 = decode)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    theta: float
    num_blocks: int
    max_blocks_per_seq: int
    num_pool_seqs: int
    script: list
    step: Tuple[StepSeq, ...]
    boost_prob: float = 0.0
    boost: float = 8.0
    block_size: int = BLOCK_SIZE
    kv_bits: int = 0          # 0: K/V cached in the storage dtype; 8 / 4: INT8 / INT4 codes + fp16 scales
    v_scale: float = 1.0      # V draws multiplied by this power of two (exact unless it overflows)

    # ---- derived sizes -------------------------------------------------
    @property
    def np_dtype(self):
        return _DTYPES[self.dtype]

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_step_tokens(self) -> int:
        return sum(s.count for s in self.step)

    @property
    def max_position(self) -> int:
        """One past the largest absolute position any fill or step writes."""
        m = 0
        for op in self.script:
            if op[0] == "fill":
                m = max(m, op[3] + op[4])
        for s in self.step:
            m = max(m, s.start + s.count)
        return m

    def fills(self):
        return [op for op in self.script if op[0] == "fill"]

    def decode_rows(self) -> List[int]:
        return [i for i, s in enumerate(self.step) if s.count == 1]

    def chunk_rows(self) -> List[int]:
        return [i for i, s in enumerate(self.step) if s.count > 1]

    # ---- random draws --------------------------------------------------
    def _rng(self, *key) -> np.random.Generator:
        return np.random.default_rng(np.random.SeedSequence(self.seed, spawn_key=key))

    def _normal(self, rng, shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        return x.astype(self.np_dtype)

    def _boost_keys(self, rng, k):
        if self.boost_prob > 0.0:
            mask = rng.random(k.shape[:2]) < self.boost_prob
            # x8 is a power of two: exact in fp16/fp32 for N(0,1) draws.
            k[mask] = k[mask] * self.np_dtype(self.boost)
        return k

    def draw_fill(self, fill_index: int) -> Tuple[np.ndarray, np.ndarray]:
        """Raw (un-rotated) K and V of fill ``fill_index``: [n][Hkv][D] each."""
        op = [o for o in self.script if o[0] == "fill" and o[1] == fill_index][0]
        n = op[4]
        rng = self._rng(1, fill_index)
        shape = (n, self.num_kv_heads, self.head_dim)
        k = self._normal(rng, shape)
        v = self._normal(rng, shape) * self.np_dtype(self.v_scale)
        return self._boost_keys(rng, k), v

    def draw_step(self, row: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Raw q [C][Hq][D], k and v [C][Hkv][D] of step row ``row``."""
        n = self.step[row].count
        rng = self._rng(2, row)
        q = self._normal(rng, (n, self.num_q_heads, self.head_dim))
        k = self._normal(rng, (n, self.num_kv_heads, self.head_dim))
        v = self._normal(rng, (n, self.num_kv_heads, self.head_dim)) * self.np_dtype(self.v_scale)
        return q, self._boost_keys(rng, k), v

    def draw_step_packed(self, rows: Sequence[int] = None, threads: int = None):
        """Step rows concatenated in order: q [T][Hq][D], k, v [T][Hkv][D]."""
        rows = list(range(len(self.step))) if rows is None else list(rows)
        parts = _parallel_map(self.draw_step, rows, threads)
        if not parts:
            z = np.zeros((0, self.num_q_heads, self.head_dim), self.np_dtype)
            zk = np.zeros((0, self.num_kv_heads, self.head_dim), self.np_dtype)
            return z, zk, zk.copy()
        return (np.concatenate([p[0] for p in parts]),
                np.concatenate([p[1] for p in parts]),
                np.concatenate([p[2] for p in parts]))


def _parallel_map(fn, items, threads=None):
    items = list(items)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if threads <= 1 or len(items) <= 1:
        return [fn(i) for i in items]
    with _cf.ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


def parallel_map(fn, items, threads=None):
    """Thread-pool map used to draw many fills at once (numpy drops the GIL)."""
    return _parallel_map(fn, items, threads)


# ---------------------------------------------------------------------------
# builders
# ---------------------------------------------------------------------------

def _blocks(n_tokens: int) -> int:
    return -(-n_tokens // BLOCK_SIZE)


def _round_robin(counts: Sequence[int], seq_ids: Sequence[int]) -> np.ndarray:
    """Order of single-block allocations: one block per sequence per round."""
    counts = np.asarray(counts, dtype=np.int64)
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    if counts.size == 0:
        return np.zeros(0, np.int64)
    rounds = int(counts.max())
    r = np.arange(rounds)[:, None]
    take = r < counts[None, :]
    return np.broadcast_to(seq_ids[None, :], take.shape)[take]


def build(name: str, seed: int, dtype: str, num_q_heads: int, num_kv_heads: int,
          head_dim: int, theta: float, seqs: Sequence[Tuple[int, int]],
          num_blocks: int = None, slack: float = 1.1,
          max_blocks_per_seq: int = None, boost_prob: float = 0.0,
          shuffle_rng: np.random.Generator = None) -> Workload:
    """Independent sequences: each (P, C) gets ceil((P+C)/16) blocks, a prefix
    fill of P tokens, and a step row (P, C).  The arena is the total plus
    ``slack`` (10 %), shuffled through the LIFO free list, allocated
    round-robin."""
    rng = shuffle_rng if shuffle_rng is not None else np.random.default_rng(seed)
    need = [_blocks(p + c) for p, c in seqs]
    total = int(sum(need))
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(slack * total)))
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(need) if need else 1
    script = [("shuffle", rng.permutation(num_blocks).astype(np.int64)),
              ("alloc", _round_robin(need, range(len(seqs))))]
    fi = 0
    for b, (p, c) in enumerate(seqs):
        if p > 0:
            script.append(("fill", fi, b, 0, p))
            fi += 1
    step = tuple(StepSeq(b, p, c) for b, (p, c) in enumerate(seqs))
    return Workload(name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, theta=theta,
                    num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq,
                    num_pool_seqs=len(seqs), script=script, step=step,
                    boost_prob=boost_prob)


# ---------------------------------------------------------------------------
# the five named workloads (one Llama-3-8B-shaped layer unless stated)
# ---------------------------------------------------------------------------

def tiny() -> Workload:
    """fp32, 1 sequence, Hq 4 / Hkv 2, D 64, 32-block arena shuffled by a seeded
    permutation, 48 cached tokens + a 16-token chunk at P=48, theta 1e4."""
    w = build("tiny_f32", 1001, "f32", 4, 2, 64, 1.0e4, [(48, 16)],
              num_blocks=32, max_blocks_per_seq=8)
    return w


def decode_batch(num_seqs: int = 64, lo: int = 512, hi: int = 4096,
                 seed: int = 1002, heads=(32, 8), name: str = "decode_llama3_8b") -> Workload:
    """64 decode tokens, contexts uniform in [512, 4096], Hq 32 / Hkv 8, D 128,
    fp16, theta 5e5, arena = total + 10 % through a shuffled LIFO list.
    ``heads`` = (Hq, Hkv): (4, 1) is one GPU's share of the layer split by
    KV head over 8 GPUs."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=num_seqs, endpoint=True)
    seqs = [(int(L) - 1, 1) for L in lens]
    return build(name, seed, "f16", heads[0], heads[1], 128, 5.0e5, seqs,
                 max_blocks_per_seq=_blocks(hi), shuffle_rng=rng)


def chunk_batch(num_seqs: int = 8, chunk: int = 512, max_prefix_blocks: int = 224,
                seed: int = 1003, heads=(32, 8), name: str = "chunk_llama3_8b") -> Workload:
    """8 sequences, cached prefix P = 16*U{0..224}, one 512-token chunk each
    (``heads`` as for decode_batch)."""
    rng = np.random.default_rng(seed)
    pre = 16 * rng.integers(0, max_prefix_blocks, size=num_seqs, endpoint=True)
    seqs = [(int(p), chunk) for p in pre]
    return build(name, seed, "f16", heads[0], heads[1], 128, 5.0e5, seqs,
                 max_blocks_per_seq=_blocks(16 * max_prefix_blocks + chunk),
                 shuffle_rng=rng)


def tp8_decode_batch() -> Workload:
    """The decode workload at one GPU's share of a KV-head split over 8 GPUs:
    Hq 4 / Hkv 1, same lengths and draws' shapes."""
    return decode_batch(heads=(4, 1), name="decode_tp8_shard")


def tp8_chunk_batch() -> Workload:
    """The chunk workload at one GPU's share of a KV-head split over 8 GPUs."""
    return chunk_batch(heads=(4, 1), name="chunk_tp8_shard")


def mixed_step(num_chunks: int = 4, chunk: int = 256, num_decodes: int = 1024,
               lo: int = 256, hi: int = 8192, num_sharers: int = 16,
               shared_prefix: int = 1024, parent_tokens: int = 1032,
               seed: int = 1004) -> Workload:
    """Continuous-batching step under a 2048-token budget: 4 chunks of 256 plus
    1024 decodes.  ``num_sharers`` decodes fork one parent holding
    ``parent_tokens`` tokens; each child's first own token lands inside the
    parent's last, partly filled block, which it copies on write.  After the
    parent is released, exactly ``shared_prefix`` tokens (whole blocks) stay
    shared by all children."""
    assert parent_tokens % BLOCK_SIZE != 0 and parent_tokens // BLOCK_SIZE * BLOCK_SIZE == shared_prefix
    rng = np.random.default_rng(seed)
    pre = 16 * rng.integers(0, (hi - chunk) // 16, size=num_chunks, endpoint=True)
    lens = rng.integers(lo, hi, size=num_decodes, endpoint=True)
    sharers = np.sort(rng.choice(num_decodes, size=num_sharers, replace=False))
    lens[sharers] = rng.integers(shared_prefix + 16, hi, size=num_sharers, endpoint=True)

    seqs = [(int(p), chunk) for p in pre] + [(int(L) - 1, 1) for L in lens]
    n_step = len(seqs)
    parent = n_step
    sharer_rows = [num_chunks + int(s) for s in sharers]
    sharer_set = set(sharer_rows)
    parent_blocks = _blocks(parent_tokens)
    cow_block = parent_blocks - 1

    need = []
    for b, (p, c) in enumerate(seqs):
        n = _blocks(p + c)
        need.append(n - parent_blocks if b in sharer_set else n)
    final_total = sum(need) + shared_prefix // BLOCK_SIZE + len(sharer_rows)
    num_blocks = int(math.ceil(1.1 * final_total))

    script = [("shuffle", rng.permutation(num_blocks).astype(np.int64)),
              ("alloc", np.full(parent_blocks, parent, np.int64)),
              ("fill", 0, parent, 0, parent_tokens)]
    for s in sharer_rows:
        script.append(("fork", s, parent))
    for s in sharer_rows:
        script.append(("cow", s, cow_block))
    script.append(("release", parent))
    script.append(("alloc", _round_robin(need, range(n_step))))
    fi = 1
    for b, (p, c) in enumerate(seqs):
        start = parent_tokens if b in sharer_set else 0
        if p > start:
            script.append(("fill", fi, b, start, p - start))
            fi += 1
    step = tuple(StepSeq(b, p, c) for b, (p, c) in enumerate(seqs))
    return Workload(name="mixed_llama3_8b", seed=seed, dtype="f16", num_q_heads=32,
                    num_kv_heads=8, head_dim=128, theta=5.0e5, num_blocks=num_blocks,
                    max_blocks_per_seq=_blocks(hi), num_pool_seqs=n_step + 1,
                    script=script, step=step)


def long_context(num_decodes: int = 32, context: int = 32768, chunk: int = 4096,
                 num_blocks: int = 68750, seed: int = 1005) -> Workload:
    """32 decodes at context 32768 plus one 4096-token chunk at P = 28672; arena
    68 750 blocks (~1.1 M tokens), fully shuffled; 1 % of key vectors x8."""
    rng = np.random.default_rng(seed)
    seqs = [(context - chunk, chunk)] + [(context - 1, 1)] * num_decodes
    return build("long_llama3_8b", seed, "f16", 32, 8, 128, 5.0e5, seqs,
                 num_blocks=num_blocks, max_blocks_per_seq=_blocks(context),
                 boost_prob=0.01, shuffle_rng=rng)


def shared_prefix_decode(num_seqs: int = 64, prefix: int = 4096, lo: int = 1, hi: int = 512,
                         seed: int = 1006) -> Workload:
    """Decodes that all continue one cached prompt (Kshipra part 3, section 3:
    many requests share a prefix such as a system prompt): a parent holding
    ``prefix`` tokens (whole blocks) is forked ``num_seqs`` times and
    released, then each child appends its own U[lo, hi] tokens and decodes
    one more.  Hq 32 / Hkv 8, D 128, fp16, theta 5e5, arena = total + 10 %."""
    assert prefix % BLOCK_SIZE == 0
    rng = np.random.default_rng(seed)
    own = rng.integers(lo, hi, size=num_seqs, endpoint=True)
    seqs = [(prefix + int(n) - 1, 1) for n in own]   # decode token at prefix + n - 1
    parent = num_seqs
    pblocks = prefix // BLOCK_SIZE
    need = [_blocks(p + c) - pblocks for p, c in seqs]
    num_blocks = int(math.ceil(1.1 * (sum(need) + pblocks)))
    script = [("shuffle", rng.permutation(num_blocks).astype(np.int64)),
              ("alloc", np.full(pblocks, parent, np.int64)),
              ("fill", 0, parent, 0, prefix)]
    for b in range(num_seqs):
        script.append(("fork", b, parent))
    script.append(("release", parent))
    script.append(("alloc", _round_robin(need, range(num_seqs))))
    for b, (p, c) in enumerate(seqs):
        if p > prefix:
            script.append(("fill", 1 + b, b, prefix, p - prefix))
    step = tuple(StepSeq(b, p, c) for b, (p, c) in enumerate(seqs))
    return Workload(name="shared_prefix_decode", seed=seed, dtype="f16", num_q_heads=32,
                    num_kv_heads=8, head_dim=128, theta=5.0e5, num_blocks=num_blocks,
                    max_blocks_per_seq=_blocks(prefix + hi), num_pool_seqs=num_seqs + 1,
                    script=script, step=step)


NAMED = {
    "tiny": tiny,
    "decode": decode_batch,
    "chunk": chunk_batch,
    "mixed": mixed_step,
    "long": long_context,
    "shared": shared_prefix_decode,
}


def named(name: str) -> Workload:
    return NAMED[name]()
