"""Runs a workload on the oracle's pool, arena, RoPE and attention.

A workload (see ``paged_kv_chunked_amd.workloads``) is random inputs plus a
pool script.  This module executes the script with ``oracle.pool`` and
``oracle.arena`` and computes the step the way the pages define it:

  append ([K3] section 4): each new token at absolute position P + t has its q
    (all query heads) and k (all KV heads) rotated at that position, rounded
    once to the storage dtype; k and v are written into the block holding
    that position; q is kept for attention.
  attention: per step row, dense masked attention over the sequence's cached
    keys (``oracle.attention``); a decode row is a one-token chunk.

Two modes: ``materialize=True`` keeps every value on the host; otherwise the
arena is symbolic and a sequence's keys are drawn and rotated only when its
rows are asked for (``sequence_kv``).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

from . import arena as _arena
from . import attention as _attention
from . import pool as _pool
from . import rope as _rope
from . import quant as _quant

STEP_SOURCE = 1 << 40     # symbolic source ids >= this are step rows


@dataclasses.dataclass
class State:
    pool: _pool.Pool
    tables: Dict[int, List[int]]
    arena: object                      # Arena or SymbolicArena
    copies: List[tuple]
    materialized: bool


def rope_tables(w, max_pos: Optional[int] = None):
    return _rope.cos_sin_table(w.theta, w.head_dim, max_pos or w.max_position)


def run_script(w, materialize: bool = True, cos_sin=None) -> State:
    p = _pool.Pool(w.num_blocks)
    tables: Dict[int, List[int]] = {s: [] for s in range(w.num_pool_seqs)}
    if not materialize:
        ar = _arena.SymbolicArena(w.num_blocks)
    elif getattr(w, "kv_bits", 0):
        ar = _arena.QuantArena(w.num_blocks, w.num_kv_heads, w.head_dim, w.kv_bits)
    else:
        ar = _arena.Arena(w.num_blocks, w.num_kv_heads, w.head_dim, w.np_dtype)
    cos, sin = cos_sin if cos_sin is not None else rope_tables(w)
    copies = []
    for op in w.script:
        kind = op[0]
        if kind == "shuffle":
            for _ in range(w.num_blocks):
                p.alloc()
            for b in op[1]:
                p.decref(int(b))
        elif kind == "alloc":
            for s in op[1]:
                tables[int(s)].append(p.alloc())
        elif kind == "fill":
            _, fi, seq, start, n = op
            if materialize:
                k, v = w.draw_fill(fi)
                pos = start + np.arange(n)
                k_rot = _rope.rotate_store(k, pos, cos, sin, w.np_dtype)
                ar.write(tables[seq], start, k_rot, v)
            else:
                ar.write(tables[seq], start, n, fi)
        elif kind == "fork":
            _, child, parent = op
            tables[child] = list(tables[parent])
            for b in tables[child]:
                p.incref(b)
        elif kind == "cow":
            _, seq, logical = op
            old = tables[seq][logical]
            new, copied = p.cow(old)
            if copied:
                ar.copy_block(old, new)
                copies.append((old, new))
            tables[seq][logical] = new
        elif kind == "release":
            for b in tables[op[1]]:
                p.decref(b)
            tables[op[1]] = []
        else:
            raise ValueError(kind)
    return State(pool=p, tables=tables, arena=ar, copies=copies, materialized=materialize)


def block_table(w, state: State) -> np.ndarray:
    """int32 [len(step)][max_blocks_per_seq], unused entries -1."""
    bt = np.full((len(w.step), w.max_blocks_per_seq), -1, dtype=np.int32)
    for r, s in enumerate(w.step):
        row = state.tables[s.seq]
        bt[r, :len(row)] = row
    return bt


def append_step(w, state: State, cos_sin=None):
    """Applies the step's append; returns the rotated q of every step row
    (storage dtype, packed [T][Hq][D] in step order)."""
    cos, sin = cos_sin if cos_sin is not None else rope_tables(w)
    qs = []
    for r, s in enumerate(w.step):
        q, k, v = w.draw_step(r)
        pos = s.start + np.arange(s.count)
        qs.append(_rope.rotate_store(q, pos, cos, sin, w.np_dtype))
        if state.materialized:
            k_rot = _rope.rotate_store(k, pos, cos, sin, w.np_dtype)
            state.arena.write(state.tables[s.seq], s.start, k_rot, v)
        else:
            state.arena.write(state.tables[s.seq], s.start, s.count, STEP_SOURCE + r)
    if not qs:
        return np.zeros((0, w.num_q_heads, w.head_dim), w.np_dtype)
    return np.concatenate(qs)


def rotated_q(w, row: int, cos_sin=None) -> np.ndarray:
    cos, sin = cos_sin if cos_sin is not None else rope_tables(w)
    s = w.step[row]
    q, _, _ = w.draw_step(row)
    return _rope.rotate_store(q, s.start + np.arange(s.count), cos, sin, w.np_dtype)


def sequence_kv(w, state: State, row: int, length: Optional[int] = None, cos_sin=None,
                codec: bool = True):
    """Stored K, V [length][Hkv][D] of step row ``row``'s sequence (after append).
    For a quantized cache these are the decoded values (fp64), or with
    ``codec=False`` the fp16 values the codec was given."""
    s = w.step[row]
    length = s.start + s.count if length is None else length
    table = state.tables[s.seq]
    if state.materialized:
        return state.arena.gather(table, length)
    cos, sin = cos_sin if cos_sin is not None else rope_tables(w)
    src, tok = state.arena.provenance(table, length)
    if (src < 0).any():
        raise ValueError("sequence reads an unwritten slot")
    K = np.empty((length, w.num_kv_heads, w.head_dim), w.np_dtype)
    V = np.empty_like(K)
    fills = {op[1]: op for op in w.script if op[0] == "fill"}
    for source in np.unique(src):
        sel = np.nonzero(src == source)[0]
        t = tok[sel]
        if source >= STEP_SOURCE:
            r = int(source - STEP_SOURCE)
            _, k, v = w.draw_step(r)
            start = w.step[r].start
        else:
            k, v = w.draw_fill(int(source))
            start = fills[int(source)][3]
        K[sel] = _rope.rotate_store(k[t], start + t, cos, sin, w.np_dtype)
        V[sel] = v[t]
    if codec and getattr(w, "kv_bits", 0):   # the cache holds the codes of these values
        return _quant.roundtrip(K, w.kv_bits), _quant.roundtrip(V, w.kv_bits)
    return K, V


def attend_row(w, state: State, row: int, q_rot: np.ndarray, scale: float,
               rows=None, heads=None, cos_sin=None) -> np.ndarray:
    """Expected fp64 output of step row ``row`` (q_rot: its [C][Hq][D] rotated q)."""
    s = w.step[row]
    K, V = sequence_kv(w, state, row, cos_sin=cos_sin)
    return _attention.attend(q_rot, K, V, s.start, scale, rows=rows, heads=heads)
