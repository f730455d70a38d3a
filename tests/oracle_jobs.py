"""Oracle work of the GPU parity tests, spread over worker processes.

The large workloads (the long-context and mixed steps) are checked on many
sequences; regenerating and rotating a 32768-token sequence and attending over
it in fp64 takes seconds per sequence on one core.  The workers are started
with the ``spawn`` method, so they never inherit the test process's GPU state;
they import only numpy, the oracle and the seeded input generators.

Each job returns, for one step row of a workload whose oracle arena is
symbolic:
  * the expected fp64 output of the requested query rows (all heads);
  * optionally SHA-256 digests of the byte images that the row's sequence's
    arena blocks must hold (K and V tiles in the library's layout, written by
    the oracle's own arena classes), for a bit-for-bit comparison of the
    blocks with a digest of the GPU's.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import multiprocessing as mp
import os

import numpy as np

from oracle import arena as oarena
from oracle import attention as oattention
from oracle import script as oscript

_W = None       # workload, symbolic oracle state, rotated queries (set per worker)
_ST = None
_Q = None


def _init(w, st, q_rot):
    global _W, _ST, _Q
    _W, _ST, _Q = w, st, q_rot


def block_images(w, K, V, nb: int):
    """Byte images (K, V) of ``nb`` blocks holding K, V [L][Hkv][D] at positions
    0..L-1 (stored fp16 values; the codec is applied for quantized caches)."""
    table = np.arange(nb)
    if w.kv_bits:
        a = oarena.QuantArena(nb, w.num_kv_heads, w.head_dim, w.kv_bits)
        a.write(table, 0, K, V)
        return a.image("k"), a.image("v")
    a = oarena.Arena(nb, w.num_kv_heads, w.head_dim, w.np_dtype)
    a.write(table, 0, K, V)
    return a.k, a.v


def digest(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _job(row: int, rows, q0: int, scale: float, want_blocks: bool):
    w, st = _W, _ST
    s = w.step[row]
    Ks, Vs = oscript.sequence_kv(w, st, row, codec=False)     # stored fp16 values
    dk = dv = None
    if want_blocks:
        nb = -(-(s.start + s.count) // w.block_size)
        ki, vi = block_images(w, Ks, Vs, nb)
        dk, dv = digest(ki), digest(vi)
    if w.kv_bits:
        K, V = oscript.sequence_kv(w, st, row)                # decoded values
    else:
        K, V = Ks, Vs
    q = _Q[q0:q0 + s.count]
    exp = oattention.attend(q, K, V, s.start, scale, rows=rows)
    return row, (None if rows is None else np.asarray(rows)), exp, dk, dv


def run(w, st, q_rot, cu, jobs, scale: float, workers: int = 8):
    """jobs: list of (row, rows or None, want_blocks).  Returns a list of
    (row, rows, expected [len(rows)][Hq][D], K digest, V digest) in job order."""
    workers = max(1, min(workers, len(jobs)))
    ctx = mp.get_context("spawn")
    env_threads = os.environ.get("OMP_NUM_THREADS")
    # each worker's BLAS gets an even share of the host's threads
    per = str(max(1, (os.cpu_count() or 16) // workers)) if env_threads is None else \
        str(max(1, int(env_threads) // workers))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
    os.environ["OMP_NUM_THREADS"] = per
    os.environ["OPENBLAS_NUM_THREADS"] = per
    try:
        with cf.ProcessPoolExecutor(workers, mp_context=ctx, initializer=_init,
                                    initargs=(w, st, q_rot)) as ex:
            futs = [ex.submit(_job, r, rows, int(cu[r]), scale, blocks) for r, rows, blocks in jobs]
            return [f.result() for f in futs]
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
