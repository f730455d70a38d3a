"""Runs a workload (``workloads.Workload``) through libpkv on one GPU.

The pool script is executed on the library's host pool (``Pool``): LIFO
allocation, reference counts and copy-on-write decisions, with the block
copies done on the device by ``pkv_copy_blocks``; cache fills go through
``kv_append_rope``.  Then ``step()`` runs the hot path on the step batch:
``kv_append_rope`` for every new token, ``paged_attention_chunk`` for the
prefill rows and ``paged_attention_decode`` for the decode rows.

Only argument preparation happens here; every value is computed by the HIP
library.  torch provides device memory and the stream.
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np

from . import (BLOCK_SIZE, DECODE_SPLIT, F16, F32, I4KV, I8KV, Pool, geom, kv_append_rope, paged_attention_chunk,
               paged_attention_chunk_plan, paged_attention_chunk_run,
               paged_attention_chunk_workspace_bytes, paged_attention_decode_shared,
               paged_attention_mixed, paged_attention_mixed_workspace_bytes,
               paged_attention_decode, paged_attention_decode_append,
               paged_attention_decode_workspace_bytes, pkv_copy_blocks,
               pkv_rope_table_bytes, pkv_rope_table_init)
from . import workloads as _wl


def _torch():
    import torch
    return torch


def default_scale(head_dim: int) -> float:
    """1/sqrt(D), rounded to fp32 (the value the kernels receive)."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def run_pool_script(w: _wl.Workload, pool: Pool, tables: Dict[int, List[int]],
                    on_fill=None, on_copy=None, on_release=None):
    """Executes the workload's pool script on the library pool, appending to
    ``tables`` (sequence -> physical block ids).  ``on_fill(op)`` is called for
    each fill, ``on_copy(src, dst)`` for each copy-on-write copy and
    ``on_release(seq)`` before a sequence's blocks are given back, in script
    order.  Returns the list of (src, dst) copies."""
    copies = []
    for op in w.script:
        kind = op[0]
        if kind == "shuffle":
            pool.alloc_n(w.num_blocks)
            for b in op[1]:
                pool.decref(int(b))
        elif kind == "alloc":
            ids = pool.alloc_n(len(op[1]))
            for s, b in zip(op[1], ids):
                tables[int(s)].append(int(b))
        elif kind == "fill":
            if on_fill is not None:
                on_fill(op)
        elif kind == "fork":
            _, child, parent = op
            tables[child] = list(tables[parent])
            for b in tables[child]:
                pool.incref(b)
        elif kind == "cow":
            _, seq, logical = op
            old = tables[seq][logical]
            new, copied = pool.cow(old)
            if copied:
                if on_copy is not None:
                    on_copy(old, new)
                copies.append((old, new))
            tables[seq][logical] = new
        elif kind == "release":
            if on_release is not None:
                on_release(op[1])
            for b in tables[op[1]]:
                pool.decref(b)
            tables[op[1]] = []
        else:
            raise ValueError(kind)
    return copies


def decode_groups(bt: np.ndarray, lens: np.ndarray, split: int = DECODE_SPLIT):
    """Groups of consecutive decode rows whose leading whole splits are the
    same physical blocks: (group_start int32 [G+1], row_skip int32 [rows]).
    A row's skip s satisfies lens > split * s (its own token comes later);
    single rows form groups with skip 0."""
    n = len(lens)
    spb = split // BLOCK_SIZE
    own = (np.asarray(lens, np.int64) - 1) // split     # whole splits before the last key
    starts, skip = [0], np.zeros(n, np.int32)
    i = 0
    while i < n:
        j, s = i + 1, int(own[i])
        while j < n and s > 0:
            same = 0
            while same < min(s, int(own[j])) and np.array_equal(
                    bt[i, same * spb:(same + 1) * spb], bt[j, same * spb:(same + 1) * spb]):
                same += 1
            if same == 0:
                break
            s = same
            j += 1
        if j - i > 1:
            skip[i:j] = s
        starts.append(j)
        i = j
    return np.asarray(starts, np.int32), skip


class DeviceWorkload:
    def __init__(self, w: _wl.Workload, device: str = "cuda", fill_batch: int = 64,
                 threads: int = 16, rope_max_pos: int = None):
        torch = _torch()
        self.w = w
        self.device = torch.device(device)
        self.tdtype = torch.float16 if w.dtype == "f16" else torch.float32
        self.kv_bits = getattr(w, "kv_bits", 0)
        self.g = geom(w.num_blocks, w.num_kv_heads, w.num_q_heads, w.head_dim,
                      I8KV if self.kv_bits == 8 else I4KV if self.kv_bits == 4
                      else F16 if w.dtype == "f16" else F32)
        self.threads = threads
        self.scale = default_scale(w.head_dim)
        N, H, D = w.num_blocks, w.num_kv_heads, w.head_dim
        x = 16 // (2 if w.dtype == "f16" else 4)   # elements per 16-byte piece of K
        if self.kv_bits:
            # INT8 / INT4 tiles: codes, then 16 fp16 scales, padded to 128-byte
            # lines; unwritten = all-ones bytes (scale NaN), as in the oracle's
            # quantized arena
            tile = (BLOCK_SIZE * D * self.kv_bits // 8 + 2 * BLOCK_SIZE + 127) // 128 * 128
            self.k_arena = torch.full((N, H, tile), 255, dtype=torch.uint8, device=self.device)
            self.v_arena = torch.full((N, H, tile), 255, dtype=torch.uint8, device=self.device)
        else:
            self._fp_arenas(N, H, D, x)
        self._finish_init(w, fill_batch, rope_max_pos)

    def _fp_arenas(self, N, H, D, x):
        torch = _torch()
        self.k_arena = torch.full((N, H, D // x, BLOCK_SIZE, x), float("nan"), dtype=self.tdtype,
                                  device=self.device)
        self.v_arena = torch.full((N, H, D, BLOCK_SIZE), float("nan"), dtype=self.tdtype,
                                  device=self.device)

    def _finish_init(self, w, fill_batch, rope_max_pos):
        torch = _torch()
        D = w.head_dim
        self.rope_max_pos = rope_max_pos or w.max_position
        nbytes = pkv_rope_table_bytes(D, self.rope_max_pos)
        self.rope = torch.empty(nbytes // 8, dtype=torch.float64, device=self.device)
        pkv_rope_table_init(self.rope, w.theta, D, self.rope_max_pos)
        self.pool = Pool(w.num_blocks)
        self.tables: Dict[int, List[int]] = {s: [] for s in range(w.num_pool_seqs)}
        self.copies = []
        self._run_script(fill_batch)
        self._prepare_step()

    # ---- pool script -----------------------------------------------------
    def _table_row(self, seq: int):
        torch = _torch()
        row = np.full((1, self.w.max_blocks_per_seq), -1, np.int32)
        t = self.tables[seq]
        row[0, :len(t)] = t
        return torch.from_numpy(row).to(self.device)

    def _append(self, seq: int, start: int, k: np.ndarray, v: np.ndarray, q=None):
        torch = _torch()
        dev = self.device
        kt = torch.from_numpy(np.ascontiguousarray(k)).to(dev)
        vt = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
        cu = torch.tensor([0, k.shape[0]], dtype=torch.int32, device=dev)
        cs = torch.tensor([start], dtype=torch.int32, device=dev)
        kv_append_rope(self.g, q, kt, vt, self.k_arena, self.v_arena, self._table_row(seq),
                       cu, cs, self.rope, self.rope_max_pos)

    def _run_script(self, fill_batch: int):
        torch = _torch()
        w = self.w
        pending = []

        def flush():
            if not pending:
                return
            draws = _wl.parallel_map(lambda op: w.draw_fill(op[1]), pending, self.threads)
            for op, (k, v) in zip(pending, draws):
                self._append(op[2], op[3], k, v)
            pending.clear()

        def on_fill(op):
            pending.append(op)
            if len(pending) >= fill_batch:
                flush()

        def on_copy(old, new):
            flush()   # fills issued before the copy must land first (stream order)
            pair = torch.tensor([[old, new]], dtype=torch.int32, device=self.device)
            pkv_copy_blocks(self.g, self.k_arena, self.v_arena, pair)

        def on_release(seq):
            # a queued fill of this sequence reads its table when flushed
            if any(op[2] == seq for op in pending):
                flush()

        self.copies = run_pool_script(w, self.pool, self.tables, on_fill=on_fill,
                                      on_copy=on_copy, on_release=on_release)
        flush()

    def block_table_host(self) -> np.ndarray:
        bt = np.full((len(self.w.step), self.w.max_blocks_per_seq), -1, np.int32)
        for r, s in enumerate(self.w.step):
            t = self.tables[s.seq]
            bt[r, :len(t)] = t
        return bt

    # ---- the step ----------------------------------------------------------
    def _prepare_step(self):
        torch = _torch()
        w, dev = self.w, self.device
        q, k, v = w.draw_step_packed(threads=self.threads)
        self.q_raw = torch.from_numpy(q).to(dev)          # as drawn (read by the append)
        self.q = torch.empty_like(self.q_raw)               # rotated queries (append output)
        self.k_new = torch.from_numpy(k).to(dev)
        self.v_new = torch.from_numpy(v).to(dev)
        counts = np.array([s.count for s in w.step], np.int64)
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        self.cu_host = cu
        self.bt_host = self.block_table_host()
        self.bt = torch.from_numpy(self.bt_host).to(dev)
        self.cu = torch.from_numpy(cu).to(dev)
        self.starts_host = np.array([s.start for s in w.step], np.int32)
        self.starts = torch.from_numpy(self.starts_host).to(dev)

        dec = w.decode_rows()
        chk = w.chunk_rows()
        # the separate decode and chunk calls need the rows of each kind to be
        # contiguous in the step; paged_attention_mixed takes any order
        self.split_ok = all(not rows or rows == list(range(rows[0], rows[-1] + 1))
                            for rows in (dec, chk))
        if not self.split_ok:
            dec, chk = [], []
        self.dec_rows, self.chunk_rows = dec, chk
        Hq, D = w.num_q_heads, w.head_dim
        if dec:
            r0, r1 = dec[0], dec[-1] + 1
            t0 = int(cu[r0])
            self.dec_tok0 = t0
            self.dec_q = self.q[t0:t0 + len(dec)]
            self.dec_bt = self.bt[r0:r1]
            lens = (self.starts_host[r0:r1] + 1).astype(np.int32)
            self.dec_lens_host = lens
            self.dec_lens = torch.from_numpy(lens).to(dev)
            self.dec_max_len = int(lens.max())
            ws = paged_attention_decode_workspace_bytes(self.g, len(dec), self.dec_max_len)
            self.dec_ws = (torch.zeros(max(ws, 4) // 4, dtype=torch.float32, device=dev)
                           if ws else None)
            self.dec_out = torch.empty((len(dec), Hq, D), dtype=torch.float32, device=dev)
            gs, skip = decode_groups(self.bt_host[r0:r1], lens)
            self.dec_group_start = torch.from_numpy(gs).to(dev)
            self.dec_row_skip = torch.from_numpy(skip).to(dev)
            self.dec_max_skip = int(skip.max()) if skip.size else 0
            self.dec_max_group = int(np.diff(gs).max()) if gs.size > 1 else 1
        if chk:
            r0, r1 = chk[0], chk[-1] + 1
            t0, t1 = int(cu[r0]), int(cu[r1])
            self.chunk_tok0 = t0
            self.chunk_q = self.q[t0:t1]
            self.chunk_bt = self.bt[r0:r1]
            self.chunk_cu = torch.from_numpy((cu[r0:r1 + 1] - t0).astype(np.int32)).to(dev)
            self.chunk_starts = self.starts[r0:r1]
            counts_c = counts[r0:r1]
            self.chunk_max_q = int(counts_c.max())
            self.chunk_max_ctx = int((self.starts_host[r0:r1] + counts_c).max())
            self.chunk_out = torch.empty((t1 - t0, Hq, D), dtype=torch.float32, device=dev)
            ws = paged_attention_chunk_workspace_bytes(self.g, r1 - r0, t1 - t0,
                                                       self.chunk_max_ctx)
            self.chunk_ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)

    def append(self, stream=None, k_arena=None, v_arena=None):
        kv_append_rope(self.g, self.q_raw, self.k_new, self.v_new,
                       self.k_arena if k_arena is None else k_arena,
                       self.v_arena if v_arena is None else v_arena,
                       self.bt, self.cu, self.starts, self.rope, self.rope_max_pos,
                       q_out=self.q, stream=stream)

    def _need_split(self):
        if not self.split_ok:
            raise ValueError("step rows of one kind must be contiguous for the separate calls")

    def decode(self, stream=None, k_arena=None, v_arena=None):
        self._need_split()
        if self.dec_rows:
            paged_attention_decode(self.g, self.dec_out, self.dec_q,
                                   self.k_arena if k_arena is None else k_arena,
                                   self.v_arena if v_arena is None else v_arena,
                                   self.dec_bt, self.dec_lens, self.dec_max_len, self.scale,
                                   self.dec_ws, stream=stream)

    def decode_shared(self, stream=None, k_arena=None, v_arena=None):
        """The decode rows through paged_attention_decode_shared (shared leading
        splits of consecutive rows read once per 4 rows)."""
        if self.dec_rows:
            paged_attention_decode_shared(self.g, self.dec_out, self.dec_q,
                                          self.k_arena if k_arena is None else k_arena,
                                          self.v_arena if v_arena is None else v_arena,
                                          self.dec_bt, self.dec_lens, self.dec_max_len, self.scale,
                                          self.dec_group_start, self.dec_row_skip,
                                          self.dec_max_skip, self.dec_max_group, self.dec_ws,
                                          stream=stream)

    def mixed(self, stream=None, k_arena=None, v_arena=None):
        """Every step row (chunks and decodes) through paged_attention_mixed,
        into ``mix_out`` [num_tokens][Hq][D] (buffers made on first use)."""
        torch = _torch()
        w = self.w
        if not hasattr(self, "mix_out"):
            counts = np.diff(self.cu_host).astype(np.int64)
            T = int(self.cu_host[-1])
            self.mix_max_q = int(counts.max())
            self.mix_max_ctx = int((self.starts_host + counts).max())
            self.mix_out = torch.empty((T, w.num_q_heads, w.head_dim), dtype=torch.float32,
                                       device=self.device)
            ws = paged_attention_mixed_workspace_bytes(self.g, len(w.step), T, self.mix_max_ctx)
            self.mix_ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=self.device)
        paged_attention_mixed(self.g, self.mix_out, self.q,
                              self.k_arena if k_arena is None else k_arena,
                              self.v_arena if v_arena is None else v_arena,
                              self.bt, self.cu, self.starts, self.mix_max_q, self.mix_max_ctx,
                              self.scale, self.mix_ws, stream=stream)

    def chunk(self, stream=None, k_arena=None, v_arena=None):
        self._need_split()
        if self.chunk_rows:
            paged_attention_chunk(self.g, self.chunk_out, self.chunk_q,
                                  self.k_arena if k_arena is None else k_arena,
                                  self.v_arena if v_arena is None else v_arena,
                                  self.chunk_bt, self.chunk_cu, self.chunk_starts,
                                  self.chunk_max_q, self.chunk_max_ctx, self.scale,
                                  self.chunk_ws, stream=stream)

    def chunk_plan(self, stream=None):
        """paged_attention_chunk_plan for the chunk rows (the schedule into
        ``chunk_ws``)."""
        self._need_split()
        if self.chunk_rows:
            paged_attention_chunk_plan(self.g, self.chunk_bt, self.chunk_cu, self.chunk_starts,
                                       self.chunk_q.shape[0], self.chunk_max_q,
                                       self.chunk_max_ctx, self.chunk_ws, stream=stream)

    def chunk_run(self, stream=None, k_arena=None, v_arena=None):
        """paged_attention_chunk_run over the schedule of the last chunk_plan()."""
        self._need_split()
        if self.chunk_rows:
            paged_attention_chunk_run(self.g, self.chunk_out, self.chunk_q,
                                      self.k_arena if k_arena is None else k_arena,
                                      self.v_arena if v_arena is None else v_arena,
                                      self.chunk_bt, self.chunk_cu, self.chunk_starts,
                                      self.chunk_max_q, self.chunk_max_ctx, self.scale,
                                      self.chunk_ws, stream=stream)

    def decode_append(self, stream=None, k_arena=None, v_arena=None):
        """The decode rows' append and attention in one paged_attention_decode_append
        call (fp16, INT8 or INT4 arenas; every step row a decode): the same q
        rotation, arena writes and outputs as append() followed by decode()."""
        self._need_split()
        if self.chunk_rows:
            raise ValueError("decode_append covers steps of decode rows only")
        if self.dec_rows:
            t0, n = self.dec_tok0, len(self.dec_rows)
            paged_attention_decode_append(self.g, self.dec_out, self.q_raw[t0:t0 + n], self.dec_q,
                                          self.k_new[t0:t0 + n], self.v_new[t0:t0 + n],
                                          self.k_arena if k_arena is None else k_arena,
                                          self.v_arena if v_arena is None else v_arena,
                                          self.dec_bt, self.dec_lens, self.dec_max_len,
                                          self.scale, self.rope, self.rope_max_pos, self.dec_ws,
                                          stream=stream)

    def step(self, stream=None, k_arena=None, v_arena=None):
        """One pass of the hot path over the step batch."""
        self.append(stream, k_arena, v_arena)
        self.chunk(stream, k_arena, v_arena)
        self.decode(stream, k_arena, v_arena)

    # ---- algorithmic work of the attention kernels --------------------------
    def decode_bytes(self) -> int:
        """Bytes decode must move: K and V of every context token (physical
        blocks shared by several sequences once), q, out, table entries, lens."""
        if not self.dec_rows:
            return 0
        w = self.w
        elt = 2 if w.dtype == "f16" else 4
        if self.kv_bits:   # codes plus the fp16 scale of each head vector
            per_tok = 2 * w.num_kv_heads * (w.head_dim * self.kv_bits // 8 + 2)
        else:
            per_tok = 2 * w.num_kv_heads * w.head_dim * elt
        seen = {}
        for r, L in zip(self.dec_rows, self.dec_lens_host):
            t = self.tables[w.step[r].seq]
            nb = -(-int(L) // BLOCK_SIZE)
            for i in range(nb):
                toks = min(BLOCK_SIZE, int(L) - i * BLOCK_SIZE)
                seen[t[i]] = max(seen.get(t[i], 0), toks)
        kv = per_tok * sum(seen.values())
        S = len(self.dec_rows)
        blocks = int(sum(-(-int(L) // BLOCK_SIZE) for L in self.dec_lens_host))
        qo = S * w.num_q_heads * w.head_dim * (elt + 4)
        return kv + qo + 4 * blocks + 4 * S

    def decode_append_bytes(self) -> int:
        """decode_bytes() plus the fused append's own traffic: the rotated
        queries written, each new key and value read and written to the arena,
        and one RoPE table row (fp64 cos, sin per pair) per sequence."""
        if not self.dec_rows:
            return 0
        w = self.w
        S = len(self.dec_rows)
        elt = 2 if w.dtype == "f16" else 4
        q_out = S * w.num_q_heads * w.head_dim * elt
        kv_new = 2 * 2 * S * w.num_kv_heads * w.head_dim * elt
        rope = S * (w.head_dim // 2) * 16
        return self.decode_bytes() + q_out + kv_new + rope

    def chunk_flops(self) -> int:
        """4 * D * Hq per visible (query, key) pair."""
        w = self.w
        pairs = 0
        for r in self.chunk_rows:
            s = w.step[r]
            pairs += s.count * s.start + s.count * (s.count + 1) // 2
        return 4 * w.head_dim * w.num_q_heads * pairs
