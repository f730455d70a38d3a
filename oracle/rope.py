"""Rotary position embedding, closed form (oracle; test infrastructure only).

[K3] section 4 "Chunked Prefill": RoPE uses absolute positions, so a chunk that
starts after P cached tokens is rotated at positions P, P+1, ... .  The pages
do not say which RoPE variant; the model they run is a Llama-style GQA model
on HF transformers, so this is the RoFormer rotation with Llama's
"rotate-half" pairing: element i is paired with element i + D/2 and the pair is
rotated by the angle  pos * theta^(-2i/D),  i in [0, D/2).

Bit-exact contract with the GPU path (both sides follow the same recipe, with
no shared code):
  * inverse frequencies and cos/sin are computed in fp64 by the C library
    (``math.pow``, ``math.cos``, ``math.sin`` here; numpy's vectorised
    transcendentals may use other implementations and are not used);
  * the rotation is evaluated in fp64 as separate products and a sum (no fused
    multiply-add), then rounded once to the storage dtype with numpy's
    round-to-nearest-even ``astype``.
"""
from __future__ import annotations

import functools
import math

import numpy as np


def inv_freq(theta: float, head_dim: int) -> np.ndarray:
    """theta^(-2i/D) for i in [0, D/2), fp64, via libm pow."""
    return np.array([math.pow(theta, -(2.0 * i) / head_dim) for i in range(head_dim // 2)],
                    dtype=np.float64)


@functools.lru_cache(maxsize=8)
def _table(theta: float, head_dim: int, max_pos: int):
    inv = inv_freq(theta, head_dim)
    half = head_dim // 2
    cos = np.empty((max_pos, half), np.float64)
    sin = np.empty((max_pos, half), np.float64)
    mc, ms = math.cos, math.sin
    for p in range(max_pos):
        fp = float(p)
        row_c = cos[p]
        row_s = sin[p]
        for i in range(half):
            a = fp * inv[i]
            row_c[i] = mc(a)
            row_s[i] = ms(a)
    cos.setflags(write=False)
    sin.setflags(write=False)
    return cos, sin


def cos_sin_table(theta: float, head_dim: int, max_pos: int):
    """(cos, sin), each fp64 [max_pos][D/2]: entry [p][i] = cos/sin(p * inv_freq[i])."""
    return _table(float(theta), int(head_dim), int(max_pos))


def rotate(x: np.ndarray, positions: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Exact-input fp64 rotation of x [n][H][D] at positions [n]; returns fp64.

    x'_i       = x_i c_i - x_{i+D/2} s_i
    x'_{i+D/2} = x_{i+D/2} c_i + x_i s_i
    """
    x64 = np.asarray(x).astype(np.float64)
    half = x64.shape[-1] // 2
    pos = np.asarray(positions, dtype=np.int64)
    c = cos[pos][:, None, :]
    s = sin[pos][:, None, :]
    a = x64[..., :half]
    b = x64[..., half:]
    lo = a * c - b * s
    hi = b * c + a * s
    return np.concatenate([lo, hi], axis=-1)


def rotate_store(x: np.ndarray, positions: np.ndarray, cos: np.ndarray, sin: np.ndarray,
                 dtype) -> np.ndarray:
    """Rotation rounded once (RNE) to the storage dtype."""
    return rotate(x, positions, cos, sin).astype(dtype)
