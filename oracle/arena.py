"""Block arena: where each token's K and V live (oracle; test infrastructure only).

[K3] section 1 "Block-Arena KV Cache": KV memory is reserved once as an arena
of fixed-size blocks; a sequence's block table maps its logical block i
(positions 16i .. 16i+15) to a physical block id.  [K3] section 4 reads the
blocks in place through that table.

Layout (the pages fix none; this is the layout the library documents):
  K arena  [num_blocks][Hkv][D/x][16][x]   x = 16 bytes of elements (8 for fp16,
           4 for fp32): element d of the key in slot s sits at [d // x][s][d % x]
  V arena  [num_blocks][Hkv][D][16]        head-dim-major inside a (block, head) tile
Position ``pos`` of a sequence with table ``bt`` lives in block ``bt[pos // 16]``,
slot ``pos % 16``.

Two forms:
  Arena          the values themselves (storage dtype), unwritten slots = NaN
  SymbolicArena  for each (block, slot) *which* append wrote it (source id,
                 token index); values are drawn and rotated on demand.  Used for
                 workloads too large to materialise on the host.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def slots(table_row, start: int, n: int):
    """Physical (block, slot) of positions start .. start+n-1."""
    pos = start + np.arange(n, dtype=np.int64)
    row = np.asarray(table_row, dtype=np.int64)
    return row[pos // BLOCK], pos % BLOCK


def piece(dtype) -> int:
    """Elements per 16-byte piece of the K layout."""
    return 16 // np.dtype(dtype).itemsize


class Arena:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype):
        x = piece(dtype)
        self.x = x
        self.k = np.full((num_blocks, num_kv_heads, head_dim // x, BLOCK, x), np.nan, dtype=dtype)
        self.v = np.full((num_blocks, num_kv_heads, head_dim, BLOCK), np.nan, dtype=dtype)

    def write(self, table_row, start: int, k_store: np.ndarray, v_store: np.ndarray) -> None:
        """k_store, v_store [n][Hkv][D] (already in the storage dtype)."""
        n, H, D = k_store.shape
        blk, slot = slots(table_row, start, n)
        self.k[blk, :, :, slot, :] = k_store.reshape(n, H, D // self.x, self.x)
        self.v[blk, :, :, slot] = v_store

    def copy_block(self, src: int, dst: int) -> None:
        self.k[dst] = self.k[src]
        self.v[dst] = self.v[src]

    def swap_out(self, ids):
        """[K3] section 5, preemption by swapping: the tiles of blocks ``ids``
        (all KV heads, all 16 slots) packed block after block, K tile then V
        tile, as raw bytes (the layout pkv_swap_out documents)."""
        out = []
        for b in ids:
            out.append(np.ascontiguousarray(self.k[b]).view(np.uint8).ravel())
            out.append(np.ascontiguousarray(self.v[b]).view(np.uint8).ravel())
        return np.concatenate(out) if out else np.zeros(0, np.uint8)

    def swap_in(self, ids, packed: np.ndarray) -> None:
        """Inverse of swap_out: tile i of ``packed`` goes back into block ids[i]."""
        kt = self.k[0].nbytes
        vt = self.v[0].nbytes
        for i, b in enumerate(ids):
            base = i * (kt + vt)
            self.k[b] = packed[base:base + kt].view(self.k.dtype).reshape(self.k.shape[1:])
            self.v[b] = packed[base + kt:base + kt + vt].view(self.v.dtype).reshape(self.v.shape[1:])

    def gather(self, table_row, length: int):
        """Dense K, V [length][Hkv][D] of one sequence (the copy the method avoids)."""
        blk, slot = slots(table_row, 0, length)
        K = self.k[blk, :, :, slot, :]                       # [L][Hkv][D/x][x]
        return K.reshape(length, K.shape[1], -1), self.v[blk, :, :, slot]


class SymbolicArena:
    """Per (block, slot): the source that wrote it and the token index inside it."""

    def __init__(self, num_blocks: int):
        self.src = np.full((num_blocks, BLOCK), -1, dtype=np.int64)
        self.tok = np.full((num_blocks, BLOCK), -1, dtype=np.int64)

    def write(self, table_row, start: int, n: int, source: int) -> None:
        blk, slot = slots(table_row, start, n)
        self.src[blk, slot] = source
        self.tok[blk, slot] = np.arange(n, dtype=np.int64)

    def copy_block(self, src: int, dst: int) -> None:
        self.src[dst] = self.src[src]
        self.tok[dst] = self.tok[src]

    def provenance(self, table_row, length: int):
        blk, slot = slots(table_row, 0, length)
        return self.src[blk, slot], self.tok[blk, slot]
