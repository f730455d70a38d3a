"""Group quantization of KV vectors (oracle; test infrastructure only).

[K3] section 2 "INT4 Quantization and the Scale Bug": values are quantized per
group with one FP16 scale per group and rounded to the nearest step, which
reconstructs every value within half a step, |x - x_hat| <= s / 2 -- but only
if encoding and decoding use the same scale.  The pages' bug encoded with the
FP32 scale and decoded with its FP16 rounding; their fix rounds the scale to
FP16 once and encodes with that value (converted back to FP32).  INT4 costs
4 + 16/128 = 4.125 bits per value with groups of 128.

The pages quantize weights; here the same codec is applied to cached K and V.
Readings (the pages leave these open):
  * group = one (token, KV head) vector of head_dim values (128 for the
    Llama-3-8B shape, the pages' group size);
  * symmetric scale from the group's largest magnitude: s = fp16(fp32(amax) /
    qmax) with qmax = 127 (INT8) or 7 (INT4), floored at the smallest positive
    fp16 value so that an all-zero group encodes as zeros;
  * the value quantized is the one an FP16 cache would hold (for k: rotated
    and rounded once to fp16);
  * encode q = round-half-even(fp32(x) / fp32(s)) (IEEE fp32 division, as
    torch's round(w / scales_for_quant)), clipped to [-qmax, qmax] (never
    reached: amax / fp16(amax / qmax) stays below qmax + 1/2);
  * decode x_hat = q * s, exact in fp64.
"""
from __future__ import annotations

import numpy as np

QMAX = {8: 127, 4: 7}
MIN_SCALE = np.float16(2.0 ** -24)   # smallest positive fp16


def scale(x: np.ndarray, bits: int) -> np.ndarray:
    """FP16 scale of every group (last axis) of fp16 values ``x``."""
    amax = np.abs(x.astype(np.float32)).max(axis=-1)
    s = (amax / np.float32(QMAX[bits])).astype(np.float16)
    return np.maximum(s, MIN_SCALE)


def encode(x: np.ndarray, bits: int = 8, s: np.ndarray = None):
    """Returns (codes int8 [..., G], scales fp16 [...]) with the scale used on
    both sides ([K3] section 2's fix)."""
    if s is None:
        s = scale(x, bits)
    q = np.rint(x.astype(np.float32) / s.astype(np.float32)[..., None])
    q = np.clip(q, -QMAX[bits], QMAX[bits]).astype(np.int8)
    return q, s


def decode(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x_hat = q * s in fp64 (exact: an 8-bit code times an 11-bit significand)."""
    return q.astype(np.float64) * s.astype(np.float64)[..., None]


def roundtrip(x: np.ndarray, bits: int = 8) -> np.ndarray:
    q, s = encode(x, bits)
    return decode(q, s)


def encode_with_fp32_scale(x: np.ndarray, bits: int = 8):
    """The pages' bug, kept for the test that shows why it broke the bound:
    codes from the FP32 scale, stored scale its FP16 rounding."""
    amax = np.abs(x.astype(np.float32)).max(axis=-1)
    s32 = np.maximum(amax / np.float32(QMAX[bits]), np.float32(MIN_SCALE))
    q = np.rint(x.astype(np.float32) / s32[..., None])
    q = np.clip(q, -QMAX[bits], QMAX[bits]).astype(np.int8)
    return q, s32.astype(np.float16)


def bits_per_value(bits: int, group: int = 128) -> float:
    """Code bits plus the group's FP16 scale spread over its values."""
    return bits + 16.0 / group
