"""Paged-KV attention for AMD MI355X (gfx950): Python binding of libpkv.

Thin ctypes layer over the C ABI declared in ``include/pkv.h``; every function
keeps the C name and only marshals arguments (torch tensors -> device
pointers, sizes, the current HIP stream).  All computation happens in the HIP
kernels of ``libpkv.so``; if the library is missing, every call raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

F16, F32, I8KV, I4KV = 0, 1, 2, 3
BLOCK_SIZE = 16
DECODE_SPLIT = 384   # tokens per decode split (fixed by the library, see pkv.h)

STATUS = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_SHAPE", 3: "PKV_ERR_DTYPE",
          4: "PKV_ERR_RANGE", 5: "PKV_ERR_WORKSPACE", 6: "PKV_ERR_NOMEM",
          7: "PKV_ERR_REFCOUNT", 8: "PKV_ERR_HIP"}


class PkvError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, code)}")
        self.code = code


class Geom(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


def geom(num_blocks: int, num_kv_heads: int, num_q_heads: int, head_dim: int,
         dtype: int = F16) -> Geom:
    return Geom(num_blocks, BLOCK_SIZE, num_kv_heads, num_q_heads, head_dim, dtype)


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PG = ctypes.POINTER(Geom)

_SIGS = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_abi_version": (_I32, []),
    "pkv_source_hash": (ctypes.c_char_p, []),
    "pkv_rope_table_bytes": (ctypes.c_int, [_I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_rope_table_host": (ctypes.c_int, [_P, ctypes.c_double, _I32, _I32]),
    "pkv_rope_table_init": (ctypes.c_int, [_P, ctypes.c_double, _I32, _I32, _P]),
    "kv_append_rope": (ctypes.c_int, [_PG, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _I32,
                                      _I32, _P, _I32, _P]),
    "paged_attention_decode_workspace_bytes": (ctypes.c_int, [_PG, _I32, _I32,
                                                              ctypes.POINTER(ctypes.c_size_t)]),
    "paged_attention_decode": (ctypes.c_int, [_PG, _P, _I32, _P, _P, _P, _P, _I32, _P, _I32,
                                              _I32, ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "paged_attention_decode_append": (ctypes.c_int, [_PG, _P, _I32, _P, _P, _P, _P, _P, _P, _P,
                                                     _I32, _P, _I32, _I32, ctypes.c_float, _P,
                                                     _I32, _P, ctypes.c_size_t, _P]),
    "paged_attention_decode_noalloc": (ctypes.c_int, [_PG, _P, _I32, _P, _P, _P, _P, _I32, _P,
                                                      _I32, _I32, ctypes.c_float, _P]),
    "paged_attention_decode_shared": (ctypes.c_int, [_PG, _P, _I32, _P, _P, _P, _P, _I32, _P,
                                                     _I32, _I32, ctypes.c_float, _P, _P, _I32,
                                                     _I32, _I32, _P, ctypes.c_size_t, _P]),
    "paged_attention_chunk_workspace_bytes": (ctypes.c_int, [_PG, _I32, _I32, _I32,
                                                             ctypes.POINTER(ctypes.c_size_t)]),
    "paged_attention_chunk_parts": (ctypes.c_int, [_PG, _I32, _I32, _I32,
                                                   ctypes.POINTER(ctypes.c_int32)]),
    "paged_attention_chunk": (ctypes.c_int, [_PG, _P, _I32, _P, _P, _P, _P, _I32, _P, _P, _I32,
                                             _I32, _I32, _I32, ctypes.c_float, _P,
                                             ctypes.c_size_t, _P]),
    "paged_attention_chunk_plan": (ctypes.c_int, [_PG, _I32, _P, _P, _I32, _I32, _I32, _I32, _P,
                                                   ctypes.c_size_t, _P]),
    "paged_attention_chunk_run": (ctypes.c_int, [_PG, _P, _I32, _P, _P, _P, _P, _I32, _P, _P,
                                                 _I32, _I32, _I32, _I32, ctypes.c_float, _P,
                                                 ctypes.c_size_t, _P]),
    "paged_attention_mixed_workspace_bytes": (ctypes.c_int, [_PG, _I32, _I32, _I32,
                                                             ctypes.POINTER(ctypes.c_size_t)]),
    "paged_attention_mixed": (ctypes.c_int, [_PG, _P, _I32, _P, _P, _P, _P, _I32, _P, _P, _I32,
                                             _I32, _I32, _I32, ctypes.c_float, _P,
                                             ctypes.c_size_t, _P]),
    "pkv_copy_blocks": (ctypes.c_int, [_PG, _P, _P, _P, _I32, _P]),
    "pkv_swap_bytes": (ctypes.c_int, [_PG, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_swap_out": (ctypes.c_int, [_PG, _P, _P, _P, _I32, _P, ctypes.c_size_t, _P]),
    "pkv_swap_in": (ctypes.c_int, [_PG, _P, _P, _P, _I32, _P, ctypes.c_size_t, _P]),
    "pkv_pool_create": (_P, [_I32]),
    "pkv_pool_destroy": (None, [_P]),
    "pkv_pool_alloc": (ctypes.c_int, [_P, _PI32]),
    "pkv_pool_alloc_n": (ctypes.c_int, [_P, _I32, _P]),
    "pkv_pool_incref": (ctypes.c_int, [_P, _I32]),
    "pkv_pool_decref": (ctypes.c_int, [_P, _I32]),
    "pkv_pool_cow": (ctypes.c_int, [_P, _I32, _PI32, _PI32]),
    "pkv_pool_num_free": (_I32, [_P]),
    "pkv_pool_refcount": (_I32, [_P, _I32]),
    "pkv_pool_free_list": (ctypes.c_int, [_P, _P, _I32, _PI32]),
    "pkv_pool_can_admit": (_I32, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
    "pkv_radix_create": (_P, [_P]),
    "pkv_radix_destroy": (None, [_P]),
    "pkv_radix_match": (_I32, [_P, _P, _I32, _P, _I32]),
    "pkv_radix_insert": (ctypes.c_int, [_P, _P, _I32, _P]),
    "pkv_radix_evict": (_I32, [_P, _I32]),
    "pkv_radix_evictable": (_I32, [_P]),
    "pkv_radix_num_nodes": (_I32, [_P]),
    "pkv_validate_tables": (ctypes.c_int, [_PG, _P, _I32, _P, _I32]),
    "pkv_f64_to_f16_host": (ctypes.c_int, [_P, _P, ctypes.c_int64]),
    "pkv_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpkv.so.  Raises if it has not been built, or if it was built
    from sources other than the ones beside it (its embedded source hash)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_chunked_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        from . import build as _build
        built, here = handle.pkv_source_hash().decode(), _build.source_hash()
        if built != here:
            raise RuntimeError(f"{LIB_PATH} was built from other sources (library "
                               f"{built[:12]}, sources {here[:12]}): rebuild it with "
                               "`python -m paged_kv_chunked_amd.build`")
        _lib = handle
    return _lib


def pkv_source_hash() -> str:
    """Hash of the sources and flags the loaded library was built from."""
    return lib().pkv_source_hash().decode()


def _check(code: int, where: str) -> None:
    if code != 0:
        raise PkvError(code, where)


# ---------------------------------------------------------------------------
# tensor marshalling helpers (torch is imported lazily: the pool and host
# helpers work without it)
# ---------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpkv must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# C ABI, same names
# ---------------------------------------------------------------------------

def pkv_abi_version() -> int:
    return lib().pkv_abi_version()


def pkv_rope_table_bytes(head_dim: int, max_pos: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().pkv_rope_table_bytes(head_dim, max_pos, ctypes.byref(n)), "pkv_rope_table_bytes")
    return n.value


def pkv_rope_table_host(out, theta: float, head_dim: int, max_pos: int) -> None:
    """out: a writable numpy float64 array of [max_pos][head_dim/2][2]."""
    _check(lib().pkv_rope_table_host(out.ctypes.data, theta, head_dim, max_pos),
           "pkv_rope_table_host")


def pkv_rope_table_init(table, theta: float, head_dim: int, max_pos: int, stream=None) -> None:
    _check(lib().pkv_rope_table_init(_ptr(table), theta, head_dim, max_pos, _stream(stream)),
           "pkv_rope_table_init")


def kv_append_rope(g: Geom, q, k, v, k_arena, v_arena, block_table, cu_q_lens, chunk_start,
                   rope_table, rope_max_pos: int, num_tokens: Optional[int] = None,
                   q_out=None, stream=None) -> None:
    """q_out=None rotates q in place."""
    num_seqs = chunk_start.shape[0]
    if num_tokens is None:
        num_tokens = k.shape[0]
    _check(lib().kv_append_rope(ctypes.byref(g), _ptr(q), _ptr(q_out), _ptr(k), _ptr(v),
                                _ptr(k_arena),
                                _ptr(v_arena), _ptr(block_table), block_table.shape[1],
                                _ptr(cu_q_lens), _ptr(chunk_start), num_seqs, num_tokens,
                                _ptr(rope_table), rope_max_pos, _stream(stream)),
           "kv_append_rope")


def paged_attention_decode_workspace_bytes(g: Geom, num_seqs: int, max_context_len: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().paged_attention_decode_workspace_bytes(ctypes.byref(g), num_seqs,
                                                        max_context_len, ctypes.byref(n)),
           "paged_attention_decode_workspace_bytes")
    return n.value


def paged_attention_decode(g: Geom, out, q, k_arena, v_arena, block_table, context_lens,
                           max_context_len: int, scale: float, workspace=None,
                           stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_decode(ctypes.byref(g), _ptr(out), F32, _ptr(q), _ptr(k_arena),
                                        _ptr(v_arena), _ptr(block_table), block_table.shape[1],
                                        _ptr(context_lens), context_lens.shape[0],
                                        max_context_len, scale, _ptr(workspace), ws_bytes,
                                        _stream(stream)),
           "paged_attention_decode")


def paged_attention_decode_append(g: Geom, out, q, q_out, k, v, k_arena, v_arena, block_table,
                                  context_lens, max_context_len: int, scale: float, rope,
                                  rope_max_pos: int, workspace=None, stream=None) -> None:
    """kv_append_rope of one new token per sequence (at position
    context_lens[b] - 1) and paged_attention_decode in one call; q_out receives
    the rotated queries and must not overlap q."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_decode_append(ctypes.byref(g), _ptr(out), F32, _ptr(q),
                                               _ptr(q_out), _ptr(k), _ptr(v), _ptr(k_arena),
                                               _ptr(v_arena), _ptr(block_table),
                                               block_table.shape[1], _ptr(context_lens),
                                               context_lens.shape[0], max_context_len, scale,
                                               _ptr(rope), rope_max_pos, _ptr(workspace),
                                               ws_bytes, _stream(stream)),
           "paged_attention_decode_append")


def paged_attention_decode_noalloc(g: Geom, out, q, k_arena, v_arena, block_table, context_lens,
                                   max_context_len: int, scale: float, stream=None) -> None:
    """paged_attention_decode without a workspace: the split partials live in
    the library's static per-GPU scratch array (calls on one GPU must not
    overlap)."""
    _check(lib().paged_attention_decode_noalloc(ctypes.byref(g), _ptr(out), F32, _ptr(q),
                                                _ptr(k_arena), _ptr(v_arena), _ptr(block_table),
                                                block_table.shape[1], _ptr(context_lens),
                                                context_lens.shape[0], max_context_len, scale,
                                                _stream(stream)),
           "paged_attention_decode_noalloc")


def paged_attention_decode_shared(g: Geom, out, q, k_arena, v_arena, block_table, context_lens,
                                  max_context_len: int, scale: float, group_start, row_skip,
                                  max_skip: int, max_group_size: int, workspace=None,
                                  stream=None) -> None:
    """paged_attention_decode with groups of rows sharing their leading splits
    (group_start: device int32 [G+1]; row_skip: device int32 [num_seqs])."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_decode_shared(
        ctypes.byref(g), _ptr(out), F32, _ptr(q), _ptr(k_arena), _ptr(v_arena),
        _ptr(block_table), block_table.shape[1], _ptr(context_lens), context_lens.shape[0],
        max_context_len, scale, _ptr(group_start), _ptr(row_skip), group_start.shape[0] - 1,
        max_skip, max_group_size, _ptr(workspace), ws_bytes, _stream(stream)),
        "paged_attention_decode_shared")


def paged_attention_chunk_workspace_bytes(g: Geom, num_seqs: int, num_tokens: int,
                                          max_context_len: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().paged_attention_chunk_workspace_bytes(ctypes.byref(g), num_seqs, num_tokens,
                                                       max_context_len, ctypes.byref(n)),
           "paged_attention_chunk_workspace_bytes")
    return n.value


def paged_attention_chunk_parts(g: Geom, num_seqs: int, num_tokens: int,
                                max_context_len: int) -> int:
    n = ctypes.c_int32()
    _check(lib().paged_attention_chunk_parts(ctypes.byref(g), num_seqs, num_tokens,
                                             max_context_len, ctypes.byref(n)),
           "paged_attention_chunk_parts")
    return n.value


def paged_attention_chunk(g: Geom, out, q, k_arena, v_arena, block_table, cu_q_lens,
                          chunk_start, max_q_len: int, max_context_len: int, scale: float,
                          workspace=None, stream=None) -> None:
    """``workspace``: a device tensor of at least
    paged_attention_chunk_workspace_bytes(...) bytes (the schedule of the
    attention kernel, and the key-range partials when the call is split);
    None makes a fresh one from torch's allocator."""
    if workspace is None:
        need = paged_attention_chunk_workspace_bytes(g, chunk_start.shape[0], q.shape[0],
                                                     max_context_len)
        if need:
            import torch
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_chunk(ctypes.byref(g), _ptr(out), F32, _ptr(q), _ptr(k_arena),
                                       _ptr(v_arena), _ptr(block_table), block_table.shape[1],
                                       _ptr(cu_q_lens), _ptr(chunk_start), chunk_start.shape[0],
                                       q.shape[0], max_q_len, max_context_len, scale,
                                       _ptr(workspace), ws_bytes, _stream(stream)),
           "paged_attention_chunk")


def paged_attention_chunk_plan(g: Geom, block_table, cu_q_lens, chunk_start, num_tokens: int,
                               max_q_len: int, max_context_len: int, workspace,
                               stream=None) -> None:
    """The schedule of paged_attention_chunk for this batch description into
    ``workspace`` (``block_table`` only gives its row length); a step plans
    once and then calls paged_attention_chunk_run per layer."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_chunk_plan(ctypes.byref(g), block_table.shape[1],
                                            _ptr(cu_q_lens), _ptr(chunk_start),
                                            chunk_start.shape[0], num_tokens, max_q_len,
                                            max_context_len, _ptr(workspace), ws_bytes,
                                            _stream(stream)),
           "paged_attention_chunk_plan")


def paged_attention_chunk_run(g: Geom, out, q, k_arena, v_arena, block_table, cu_q_lens,
                              chunk_start, max_q_len: int, max_context_len: int, scale: float,
                              workspace, stream=None) -> None:
    """paged_attention_chunk over the schedule that the last
    paged_attention_chunk_plan call with the same batch left in ``workspace``."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_chunk_run(ctypes.byref(g), _ptr(out), F32, _ptr(q),
                                           _ptr(k_arena), _ptr(v_arena), _ptr(block_table),
                                           block_table.shape[1], _ptr(cu_q_lens),
                                           _ptr(chunk_start), chunk_start.shape[0], q.shape[0],
                                           max_q_len, max_context_len, scale, _ptr(workspace),
                                           ws_bytes, _stream(stream)),
           "paged_attention_chunk_run")


def paged_attention_mixed_workspace_bytes(g: Geom, num_seqs: int, num_tokens: int,
                                          max_context_len: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().paged_attention_mixed_workspace_bytes(ctypes.byref(g), num_seqs, num_tokens,
                                                       max_context_len, ctypes.byref(n)),
           "paged_attention_mixed_workspace_bytes")
    return n.value


def paged_attention_mixed(g: Geom, out, q, k_arena, v_arena, block_table, cu_q_lens,
                          chunk_start, max_q_len: int, max_context_len: int, scale: float,
                          workspace=None, stream=None) -> None:
    """One varlen batch of prefill chunks and decodes (sequences of one row) in
    one attention launch; arguments as paged_attention_chunk.  ``workspace``:
    a device tensor of at least paged_attention_mixed_workspace_bytes(...)
    bytes; None makes a fresh one from torch's allocator."""
    if workspace is None:
        need = paged_attention_mixed_workspace_bytes(g, chunk_start.shape[0], q.shape[0],
                                                     max_context_len)
        if need:
            import torch
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attention_mixed(ctypes.byref(g), _ptr(out), F32, _ptr(q), _ptr(k_arena),
                                       _ptr(v_arena), _ptr(block_table), block_table.shape[1],
                                       _ptr(cu_q_lens), _ptr(chunk_start), chunk_start.shape[0],
                                       q.shape[0], max_q_len, max_context_len, scale,
                                       _ptr(workspace), ws_bytes, _stream(stream)),
           "paged_attention_mixed")


def pkv_copy_blocks(g: Geom, k_arena, v_arena, src_dst, stream=None) -> None:
    _check(lib().pkv_copy_blocks(ctypes.byref(g), _ptr(k_arena), _ptr(v_arena), _ptr(src_dst),
                                 src_dst.shape[0], _stream(stream)), "pkv_copy_blocks")


def pkv_stream_read(src, sink, stream=None) -> None:
    """Measurement helper: one streaming read of the device tensor src (its
    bytes, a multiple of 16) on the stream; sink: a device tensor of at least 4
    bytes."""
    _check(lib().pkv_stream_read(_ptr(src), _nbytes(src), _ptr(sink), _stream(stream)),
           "pkv_stream_read")


def pkv_swap_bytes(g: Geom, n: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().pkv_swap_bytes(ctypes.byref(g), n, ctypes.byref(out)), "pkv_swap_bytes")
    return out.value


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def pkv_swap_out(g: Geom, k_arena, v_arena, ids, buf, stream=None) -> None:
    """Blocks ids (device int32 [n]) -> buf (pinned host or device tensor of
    pkv_swap_bytes(n) bytes)."""
    _check(lib().pkv_swap_out(ctypes.byref(g), _ptr(k_arena), _ptr(v_arena), _ptr(ids),
                              ids.shape[0], _ptr(buf), _nbytes(buf), _stream(stream)),
           "pkv_swap_out")


def pkv_swap_in(g: Geom, k_arena, v_arena, ids, buf, stream=None) -> None:
    _check(lib().pkv_swap_in(ctypes.byref(g), _ptr(k_arena), _ptr(v_arena), _ptr(ids),
                             ids.shape[0], _ptr(buf), _nbytes(buf), _stream(stream)),
           "pkv_swap_in")


def pkv_validate_tables(g: Geom, block_table_host, lens_host) -> None:
    """Host (numpy int32) copies of a block table [S][max_blocks] and lengths [S]."""
    _check(lib().pkv_validate_tables(ctypes.byref(g), block_table_host.ctypes.data,
                                     block_table_host.shape[1], lens_host.ctypes.data,
                                     lens_host.shape[0]), "pkv_validate_tables")


def pkv_f64_to_f16_host(x, out) -> None:
    """x: numpy float64 array; out: numpy uint16 array of the same size."""
    _check(lib().pkv_f64_to_f16_host(x.ctypes.data, out.ctypes.data, x.size),
           "pkv_f64_to_f16_host")


class Pool:
    """The library's host block pool (pkv_pool_*): LIFO free list, refcounts, CoW."""

    def __init__(self, num_blocks: int):
        self._h = lib().pkv_pool_create(num_blocks)
        if not self._h:
            raise PkvError(4, "pkv_pool_create")
        self.num_blocks = num_blocks

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.pkv_pool_destroy(h)

    def alloc(self) -> int:
        out = ctypes.c_int32()
        _check(lib().pkv_pool_alloc(self._h, ctypes.byref(out)), "pkv_pool_alloc")
        return out.value

    def alloc_n(self, n: int):
        import numpy as np
        ids = np.empty(n, np.int32)
        _check(lib().pkv_pool_alloc_n(self._h, n, ids.ctypes.data), "pkv_pool_alloc_n")
        return ids

    def incref(self, b: int) -> None:
        _check(lib().pkv_pool_incref(self._h, b), "pkv_pool_incref")

    def decref(self, b: int) -> None:
        _check(lib().pkv_pool_decref(self._h, b), "pkv_pool_decref")

    def cow(self, b: int):
        out, copied = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pkv_pool_cow(self._h, b, ctypes.byref(out), ctypes.byref(copied)),
               "pkv_pool_cow")
        return out.value, bool(copied.value)

    @property
    def num_free(self) -> int:
        return lib().pkv_pool_num_free(self._h)

    def refcount(self, b: int) -> int:
        return lib().pkv_pool_refcount(self._h, b)

    def can_admit(self, evictable: int, active_reserved: int, new_need: int) -> bool:
        r = lib().pkv_pool_can_admit(self._h, evictable, active_reserved, new_need)
        if r < 0:
            raise PkvError(4, "pkv_pool_can_admit")
        return bool(r)

    def free_list(self):
        import numpy as np
        n = ctypes.c_int32()
        _check(lib().pkv_pool_free_list(self._h, None, 0, ctypes.byref(n)), "pkv_pool_free_list")
        out = np.empty(n.value, np.int32)
        _check(lib().pkv_pool_free_list(self._h, out.ctypes.data, n.value, ctypes.byref(n)),
               "pkv_pool_free_list")
        return out


class Radix:
    """The library's radix-tree prefix cache (pkv_radix_*) over a Pool."""

    def __init__(self, pool: "Pool"):
        self.pool = pool  # keeps the pool alive for the tree's lifetime
        self._h = lib().pkv_radix_create(pool._h)
        if not self._h:
            raise PkvError(1, "pkv_radix_create")

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.pkv_radix_destroy(h)

    def match(self, tokens):
        import numpy as np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        cap = t.size // BLOCK_SIZE
        out = np.empty(max(cap, 1), np.int32)
        m = lib().pkv_radix_match(self._h, t.ctypes.data, t.size, out.ctypes.data, cap)
        if m < 0:
            raise PkvError(4, "pkv_radix_match")
        return out[:m].copy()

    def insert(self, tokens, blocks) -> None:
        import numpy as np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        b = np.ascontiguousarray(blocks, dtype=np.int32)
        if b.size < t.size // BLOCK_SIZE:
            raise ValueError("one block id per whole block of tokens")
        _check(lib().pkv_radix_insert(self._h, t.ctypes.data, t.size, b.ctypes.data),
               "pkv_radix_insert")

    def evict(self, target: int) -> int:
        r = lib().pkv_radix_evict(self._h, target)
        if r < 0:
            raise PkvError(4, "pkv_radix_evict")
        return r

    def evictable(self) -> int:
        return lib().pkv_radix_evictable(self._h)

    @property
    def num_nodes(self) -> int:
        return lib().pkv_radix_num_nodes(self._h)
