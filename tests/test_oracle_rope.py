"""Pins for oracle.rope (CPU only).

The oracle's RoPE is pinned by things other than itself:
  * position 0 is the identity, exactly;
  * head_dim 2 is a plain 2-D rotation by `pos` radians (complex exponential);
  * the complex-number form of RoFormer's rotation with frequencies from
    exp/log (a different computation route) for any head_dim;
  * HF transformers' Llama `apply_rotary_pos_emb` (the routine the pages' model
    runs on) fed with the same cos/sin: pins the rotate-half pairing and signs;
  * HF's Llama rotary inverse frequencies: pins theta^(-2i/D);
  * rotation invariants: per-pair norm, and <R_m q, R_n k> = <q, R_{n-m} k>;
  * the single rounding to fp16 / fp32 against exact rational rounding.
"""
import cmath
import fractions
import math

import numpy as np
import pytest

from oracle import rope


def _rand(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def test_position_zero_is_identity():
    cos, sin = rope.cos_sin_table(1.0e4, 64, 4)
    x = _rand((3, 2, 64)).astype(np.float32)
    out = rope.rotate(x, np.zeros(3, np.int64), cos, sin)
    assert np.array_equal(out, x.astype(np.float64))


def test_head_dim_two_is_plain_rotation():
    cos, sin = rope.cos_sin_table(1.0e4, 2, 200)
    x = _rand((200, 1, 2))
    pos = np.arange(200)
    out = rope.rotate(x, pos, cos, sin)
    for p in range(200):
        z = complex(x[p, 0, 0], x[p, 0, 1]) * cmath.exp(1j * p)
        assert abs(out[p, 0, 0] - z.real) < 1e-12 and abs(out[p, 0, 1] - z.imag) < 1e-12


@pytest.mark.parametrize("D,theta", [(8, 1.0e4), (64, 1.0e4), (128, 5.0e5)])
def test_complex_form(D, theta):
    max_pos = 3000
    cos, sin = rope.cos_sin_table(theta, D, max_pos)
    rng = np.random.default_rng(D)
    pos = rng.integers(0, max_pos, size=50)
    x = rng.standard_normal((50, 3, D))
    out = rope.rotate(x, pos, cos, sin)
    half = D // 2
    for t in range(50):
        for h in range(3):
            for i in range(half):
                w = math.exp(-(2.0 * i / D) * math.log(theta))
                z = complex(x[t, h, i], x[t, h, i + half]) * cmath.exp(1j * pos[t] * w)
                # angles reach ~3000 rad: the exp/log frequency differs in the
                # last bits, which the angle magnifies by pos
                tol = 1e-12 + 4e-16 * pos[t] * abs(z)
                assert abs(out[t, h, i] - z.real) <= tol
                assert abs(out[t, h, i + half] - z.imag) <= tol


def test_matches_hf_llama_rotate_half():
    torch = pytest.importorskip("torch")
    llama = pytest.importorskip("transformers.models.llama.modeling_llama")
    D, theta, max_pos = 128, 5.0e5, 600
    cos, sin = rope.cos_sin_table(theta, D, max_pos)
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 4, 37, D))
    k = rng.standard_normal((1, 2, 37, D))
    pos = rng.integers(0, max_pos, size=37)
    c = torch.from_numpy(np.concatenate([cos[pos], cos[pos]], -1))[None]
    s = torch.from_numpy(np.concatenate([sin[pos], sin[pos]], -1))[None]
    qh, kh = llama.apply_rotary_pos_emb(torch.from_numpy(q), torch.from_numpy(k), c, s)
    qo = rope.rotate(q[0].transpose(1, 0, 2), pos, cos, sin).transpose(1, 0, 2)
    ko = rope.rotate(k[0].transpose(1, 0, 2), pos, cos, sin).transpose(1, 0, 2)
    np.testing.assert_allclose(qo, qh[0].numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(ko, kh[0].numpy(), rtol=0, atol=1e-13)


def test_inv_freq_matches_hf_llama():
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers")
    for D, theta in [(64, 1.0e4), (128, 5.0e5)]:
        cfg = tr.LlamaConfig(hidden_size=D * 4, num_attention_heads=4, head_dim=D,
                             rope_theta=theta, max_position_embeddings=4096)
        emb = tr.models.llama.modeling_llama.LlamaRotaryEmbedding(config=cfg)
        hf = emb.inv_freq.double().numpy()
        ours = rope.inv_freq(theta, D)
        np.testing.assert_allclose(ours, hf, rtol=1e-6, atol=0)   # HF builds it in fp32
        assert ours[0] == 1.0


def test_pair_norm_preserved():
    D = 128
    cos, sin = rope.cos_sin_table(5.0e5, D, 5000)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 2, D))
    pos = rng.integers(0, 5000, size=40)
    out = rope.rotate(x, pos, cos, sin)
    h = D // 2
    n0 = x[..., :h] ** 2 + x[..., h:] ** 2
    n1 = out[..., :h] ** 2 + out[..., h:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)


def test_relative_position_property():
    """<R_m q, R_n k> depends only on n - m: shifting both by d changes nothing."""
    D = 64
    cos, sin = rope.cos_sin_table(1.0e4, D, 4000)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for m, n, d in [(0, 5, 100), (17, 3, 900), (250, 1000, 2500)]:
        a = rope.rotate(q, [m], cos, sin).ravel() @ rope.rotate(k, [n], cos, sin).ravel()
        b = rope.rotate(q, [m + d], cos, sin).ravel() @ rope.rotate(k, [n + d], cos, sin).ravel()
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def _exact_round_f16(x: float) -> int:
    """Correct IEEE binary16 round-to-nearest-even of a finite double, as bits,
    by exact rational arithmetic (independent of numpy)."""
    fr = fractions.Fraction(x)
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(fr)
    if a == 0:
        return sign
    e = math.floor(math.log2(a)) if a > 0 else 0
    while fractions.Fraction(2) ** e > a:
        e -= 1
    while fractions.Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)                               # subnormal range shares 2^-14
    ulp = fractions.Fraction(2) ** (e - 10)
    m = a / ulp
    n = math.floor(m)
    rem = m - n
    if rem > fractions.Fraction(1, 2) or (rem == fractions.Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n == 2048:                                 # rounded up to the next binade
        n, e = 1024, e + 1
    if e > 15:
        return sign | 0x7C00                      # overflow to infinity
    if n < 1024:                                  # subnormal (e == -14)
        return sign | n
    return sign | ((e + 15) << 10) | (n - 1024)


def test_store_rounding_fp16_is_single_rne():
    rng = np.random.default_rng(5)
    cases = [1 + 2.0 ** -11 + 2.0 ** -40, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0, 65519.99,
             65520.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 + 2.0 ** -60, 3 * 2.0 ** -25,
             6.1e-5, 2.0 ** -14 - 2.0 ** -25, -0.0, -(1 + 2.0 ** -11)]
    bits = rng.integers(0, 2 ** 63, size=3000, dtype=np.uint64)
    rnd = bits.view(np.float64)
    rnd = rnd[np.isfinite(rnd) & (np.abs(rnd) < 7e4) & (np.abs(rnd) > 1e-9)]
    mant = rng.integers(0, 2 ** 11, size=2000)
    ties = (1.0 + (2 * mant + 1) * 2.0 ** -12) * 2.0 ** rng.integers(-20, 15, size=2000)
    vals = np.concatenate([np.array(cases), rnd, ties, rng.standard_normal(3000) * 3])
    got = vals.astype(np.float16).view(np.uint16)
    for v, g in zip(vals, got):
        assert _exact_round_f16(float(v)) == int(g), v


def test_store_rounding_fp32_is_rne():
    x = np.array([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 1 + 2.0 ** -24 + 2.0 ** -50])
    got = x.astype(np.float32)
    assert got[0] == np.float32(1.0)
    assert got[1] == np.float32(1 + 2.0 ** -22)
    assert got[2] == np.float32(1 + 2.0 ** -23)
