"""Attention over a sequence's cached keys, by the plain definition (oracle).

[K3] section 4 "Chunked Prefill" states that merging per-block partial
softmaxes (the online-softmax loop over blocks read in place) is mathematically
identical to dense masked attention.  The oracle is therefore the dense
definition itself, with nothing blocked, merged or fused:

  * gather K, V of the sequence densely (the copy the method avoids);
  * scores S[i, j] = (q_i . k_j) * scale in fp64;
  * causal mask: the row at absolute position P + i sees keys j <= P + i, i.e.
    the whole cached prefix and the chunk up to and including itself
    ([K3] section 4 says "earlier tokens in its own chunk"; it also claims
    equality with dense masking, and a decode token attends to the cache that
    already holds its own key, [K2] section 1 — so the row sees itself);
  * two-pass softmax in fp64: m = max_j S, e = exp(S - m), l = sum e, A = e / l;
  * out = A @ V in fp64.

Grouped-query attention ([K3] introduction: Llama-style model with GQA):
query head h reads KV head h // (Hq / Hkv), the contiguous grouping of HF's
``repeat_kv``.  A decode token is a chunk of one row at P = length - 1.

Score matrices are materialised for at most ``ROW_BLOCK`` rows at a time only
to bound host memory; each row is computed independently, so this changes
nothing in the arithmetic.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, start: int, scale: float,
           rows=None, heads=None) -> np.ndarray:
    """q [C][Hq][D]; K, V [L][Hkv][D] with L >= start + C (stored values).

    Returns fp64 [len(rows)][len(heads)][D]; ``rows`` / ``heads`` select a subset
    (default: all)."""
    C, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    rows = np.arange(C) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    q64 = np.asarray(q).astype(np.float64)
    out = np.empty((rows.size, len(heads), D), np.float64)
    kv64 = {}   # KV head -> its keys and values in fp64 (converted once per head group)
    for hi, h in enumerate(heads):
        g = h // G
        if g not in kv64:
            kv64 = {g: (np.asarray(K[:, g, :]).astype(np.float64),
                        np.asarray(V[:, g, :]).astype(np.float64))}
        Kg, Vg = kv64[g]
        for r0 in range(0, rows.size, ROW_BLOCK):
            r = rows[r0:r0 + ROW_BLOCK]
            pos = start + r                                   # absolute positions
            n_keys = int(pos.max()) + 1
            S = (q64[r, h, :] @ Kg[:n_keys].T) * scale        # [rows][keys]
            j = np.arange(n_keys)
            S[j[None, :] > pos[:, None]] = -np.inf            # causal mask
            m = S.max(axis=1, keepdims=True)
            e = np.exp(S - m)
            l = e.sum(axis=1, keepdims=True)
            A = e / l
            out[r0:r0 + r.size, hi, :] = A @ Vg[:n_keys]
    return out


def attend_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, length: int,
                  scale: float) -> np.ndarray:
    """One decode token (q [Hq][D]) at position length-1 over ``length`` keys."""
    return attend(q[None], K[:length], V[:length], length - 1, scale)[0]
