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


def quant_tile_size(head_dim: int, bits: int = 8) -> int:
    """Bytes of one (block, head) tile: the 16 * D codes (bits each) + 16 fp16
    scales, rounded up to whole 128-byte lines (the library's layout)."""
    return (16 * head_dim * bits // 8 + 32 + 127) // 128 * 128


def k4_record(slot):
    """INT4 K: index of the 8-byte record of the key in ``slot`` among the 16
    of a 16-dim piece (the library's layout): 2 r + u with r = 4 ((s >> 3) & 1)
    + (s & 3) and u = (s >> 2) & 1, so the two keys one lane of the decode
    kernel reads (u = 0, 1) are adjacent."""
    slot = np.asarray(slot)
    return 2 * (4 * ((slot >> 3) & 1) + (slot & 3)) + ((slot >> 2) & 1)


def v4_byte(d, slot, head_dim: int):
    """INT4 V: offset of the byte holding head dim ``d`` of the key in
    ``slot`` (the library's layout, see QuantArena); its nibble is the high
    one when (slot >> 2) & 1."""
    d, slot = np.asarray(d), np.asarray(slot)
    j = d >> 6
    G = np.where(head_dim - 64 * j >= 64, 4, 2)
    return 512 * j + 4 * (((slot >> 3) * 16 + (d & 15)) * G + ((d >> 4) & 3)) + (slot & 3)


def kpos(slot):
    """Stored position of the key in ``slot`` among the 16 of a K piece: bits
    2 and 3 exchanged (the library's layout)."""
    slot = np.asarray(slot)
    return (slot & 3) | ((slot >> 1) & 4) | ((slot << 1) & 8)


class QuantArena:
    """Arena of group-quantized K/V ([K3] section 2's codec applied per (token,
    KV head) vector, see quant.py).  Codes and scales are kept apart here, in
    slot order; the byte image of a (block, head) tile (``tile_bytes``,
    ``image``) follows the library's documented layout, quant_tile_size bytes:
      K tile  int8 codes [D/16][16][16] (16-byte pieces of 16 dims; the key of
              slot s at position kpos(s)), then 16 fp16 scales (slot order)
      V tile  int8 codes [D][16] (head-dim-major, slot order), then 16 fp16
              scales
      then padding up to the tile size (never written: all-ones bytes).
    With 4 bits, codes are packed two per byte (low nibble first, each the
    code's two's-complement low 4 bits):
      K tile  [D/16][16 records of 8 bytes] (record k4_record(s) of slot s;
              byte i holds dims 16p + i and 16p + 8 + i), then 16 fp16 scales
      V tile  head dims in groups of 64 (the last of 32 when D is not a
              multiple of 64); group j of G 16-dim blocks is [half h][d & 15]
              [block (d >> 4) & 3] words of 4 bytes at 512 j + 4 ((16 h +
              (d & 15)) G + ((d >> 4) & 3)) (v4_byte); byte i of the word of
              half h holds slots 8h + i (low nibble) and 8h + 4 + i (high),
              so 8 consecutive slots are 4 bytes in order; then 16 fp16
              scales
    Unwritten slots hold all-ones bytes (code -1, scale NaN), so a read of one
    is NaN."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, bits: int = 8):
        self.bits = bits
        H, D = num_kv_heads, head_dim
        self.kq = np.full((num_blocks, H, D // 16, BLOCK, 16), -1, np.int8)
        self.vq = np.full((num_blocks, H, D, BLOCK), -1, np.int8)
        self.ks = np.full((num_blocks, H, BLOCK), 0xFFFF, np.uint16).view(np.float16)
        self.vs = np.full((num_blocks, H, BLOCK), 0xFFFF, np.uint16).view(np.float16)

    def write(self, table_row, start: int, k_store: np.ndarray, v_store: np.ndarray) -> None:
        """k_store, v_store [n][Hkv][D] fp16 (what an fp16 cache would hold)."""
        from . import quant
        n, H, D = k_store.shape
        blk, slot = slots(table_row, start, n)
        kq, ks = quant.encode(k_store, self.bits)
        vq, vs = quant.encode(v_store, self.bits)
        self.kq[blk, :, :, slot, :] = kq.reshape(n, H, D // 16, 16)
        self.ks[blk, :, slot] = ks
        self.vq[blk, :, :, slot] = vq
        self.vs[blk, :, slot] = vs

    def copy_block(self, src: int, dst: int) -> None:
        for a in (self.kq, self.vq, self.ks, self.vs):
            a[dst] = a[src]

    def gather(self, table_row, length: int):
        """Dequantized K, V [length][Hkv][D] in fp64."""
        from . import quant
        blk, slot = slots(table_row, 0, length)
        kq = self.kq[blk, :, :, slot, :].reshape(length, self.kq.shape[1], -1)
        return (quant.decode(kq, self.ks[blk, :, slot]),
                quant.decode(self.vq[blk, :, :, slot], self.vs[blk, :, slot]))

    def swap_out(self, ids):
        """[K3] section 5 swapping: per block, the K tiles then the V tiles as
        bytes (every head's tile image: codes, 16 scales, padding)."""
        out = []
        for b in ids:
            out.append(self.tile_bytes("k", b))
            out.append(self.tile_bytes("v", b))
        return np.concatenate(out) if out else np.zeros(0, np.uint8)

    def image(self, which: str, blocks=None) -> np.ndarray:
        """Byte image [N][Hkv][tile] of the K or V arena (of ``blocks`` only if
        given)."""
        q, sc = (self.kq, self.ks) if which == "k" else (self.vq, self.vs)
        if blocks is not None:
            q, sc = q[blocks], sc[blocks]
        N, H = q.shape[:2]
        D = q.shape[2] * 16 if which == "k" else q.shape[2]
        if self.bits == 8:
            if which == "k":                # slot s to position kpos(s)
                q = q[:, :, :, np.argsort(kpos(np.arange(BLOCK))), :]
            codes = np.ascontiguousarray(q).reshape(N, H, -1).view(np.uint8)
        else:
            nib = q.view(np.uint8) & 0x0F   # two's-complement low 4 bits
            if which == "k":                # [piece][record][byte i]: dims i, 8 + i
                rec = nib[:, :, :, np.argsort(k4_record(np.arange(BLOCK))), :]
                packed = rec[..., :8] | (rec[..., 8:] << 4)
            else:                           # word of (dim, half h): byte i = slots 8h + i, 8h + 4 + i
                n = nib.reshape(nib.shape[:-1] + (2, 2, 4))     # [N][H][D][h][hi][i]
                words = n[..., 0, :] | (n[..., 1, :] << 4)      # [N][H][D][h][i]
                blocks = words.reshape(N, H, D // 16, 16, 2, 4)  # [N][H][db][d & 15][h][i]
                groups = [blocks[:, :, b0:b0 + 4].transpose(0, 1, 4, 3, 2, 5).reshape(N, H, -1)
                          for b0 in range(0, D // 16, 4)]       # [h][d & 15][db & 3][i]
                packed = np.concatenate(groups, axis=2)
            codes = np.ascontiguousarray(packed).reshape(N, H, -1)
        scales = np.ascontiguousarray(sc).view(np.uint8).reshape(N, H, -1)
        pad = quant_tile_size(D, self.bits) - codes.shape[2] - scales.shape[2]
        return np.concatenate([codes, scales, np.full((N, H, pad), 0xFF, np.uint8)], axis=2)

    def tile_bytes(self, which: str, block: int) -> np.ndarray:
        """Byte image of every head's tile of ``block`` (K or V), heads in order."""
        return self.image(which, [block]).ravel()


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
