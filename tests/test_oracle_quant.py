"""Pins of the oracle's group-quantization codec (oracle/quant.py) and of the
quantized arena, against what Kshipra part 3, section 2 fixes: one FP16 scale
per group used to encode and to decode, rounding to the nearest step, the
reconstruction bound |x - x_hat| <= s / 2, the failure of that bound when the
codes come from the FP32 scale (the pages' bug, about |q| * 2^-11 * s beyond
s / 2), and the cost of 4 + 16/128 = 4.125 bits per value (about 26% of FP16)
for INT4 with groups of 128."""
import numpy as np
import pytest

from oracle import arena, quant


def _groups(rng, n, d=128):
    x = rng.standard_normal((n, d)).astype(np.float32)
    x[rng.random((n, d)) < 0.01] *= 8.0           # heavy tail, as the long workload's keys
    return x.astype(np.float16)


@pytest.mark.parametrize("bits", [8, 4])
def test_reconstruction_bound(bits):
    x = _groups(np.random.default_rng(1), 4000)
    q, s = quant.encode(x, bits)
    err = np.abs(x.astype(np.float64) - quant.decode(q, s))
    half = s.astype(np.float64)[:, None] / 2
    assert (err <= half).all()
    assert np.abs(q).max() == quant.QMAX[bits]     # the largest value maps to the top code


@pytest.mark.parametrize("bits", [8, 4])
def test_codes_are_the_nearest_step_brute_force(bits):
    """Every code is the integer step nearest x / s (ties to even), checked by
    trying all codes."""
    rng = np.random.default_rng(2)
    x = _groups(rng, 40, d=16)
    q, s = quant.encode(x, bits)
    qmax = quant.QMAX[bits]
    cand = np.arange(-qmax, qmax + 1, dtype=np.float64)
    for g in range(x.shape[0]):
        r = x[g].astype(np.float32) / s[g].astype(np.float32)   # the fp32 quotient
        d = np.abs(r.astype(np.float64)[:, None] - cand[None, :])
        best = d.min(axis=1)
        for i in range(x.shape[1]):
            winners = cand[d[i] == best[i]]
            expect = winners[0] if winners.size == 1 else winners[winners % 2 == 0][0]
            assert q[g, i] == expect


def test_fp32_scale_breaks_the_bound_by_the_pages_margin():
    """The pages' bug: codes from the FP32 scale, decoding with its FP16
    rounding.  The bound fails, by at most |q| * 2^-11 * s (about 0.06 s for
    INT8); encoding with the FP16 scale (the fix) keeps it."""
    x = _groups(np.random.default_rng(3), 4000)
    qb, sb = quant.encode_with_fp32_scale(x, 8)
    s64 = sb.astype(np.float64)[:, None]
    err = np.abs(x.astype(np.float64) - quant.decode(qb, sb))
    assert (err > s64 / 2).any()
    excess = (err - s64 / 2) / s64
    assert excess.max() <= 127 * 2.0 ** -11 * 1.01
    assert excess.max() > 0.02
    q, s = quant.encode(x, 8)
    assert (np.abs(x.astype(np.float64) - quant.decode(q, s)) <= s.astype(np.float64)[:, None] / 2).all()


def test_bits_per_value_from_the_pages():
    assert quant.bits_per_value(4, 128) == 4.125
    assert abs(quant.bits_per_value(4, 128) / 16 - 0.26) < 0.005
    assert quant.bits_per_value(8, 128) == 8.125


def test_special_groups():
    # all zeros: zero codes, exact zeros back
    z = np.zeros((1, 128), np.float16)
    q, s = quant.encode(z)
    assert (q == 0).all() and (quant.decode(q, s) == 0).all()
    # a group whose scale is exact: amax = 127 * 2^-3 gives s = 2^-3 and every
    # multiple of 2^-3 in range reconstructs exactly
    x = (np.arange(-127, 129, 2)[:128] * 0.125).astype(np.float16)[None]
    x[0, 0] = np.float16(-127 * 0.125)
    q, s = quant.encode(x)
    assert s[0] == np.float16(0.125)
    assert np.array_equal(quant.decode(q, s)[0], x[0].astype(np.float64))
    # a single non-zero value: top code, reconstructed within half a step
    y = np.zeros((1, 128), np.float16)
    y[0, 5] = np.float16(-3.3)
    q, s = quant.encode(y)
    assert q[0, 5] == -127 and abs(quant.decode(q, s)[0, 5] - float(y[0, 5])) <= float(s[0]) / 2


def test_quant_arena_gather_is_codec_roundtrip_and_tile_size():
    rng = np.random.default_rng(4)
    H, D = 2, 32
    a = arena.QuantArena(6, H, D)
    k = _groups(rng, 20 * H, D).reshape(20, H, D)
    v = _groups(rng, 20 * H, D).reshape(20, H, D)
    table = [4, 1]
    a.write(table, 0, k, v)
    K, V = a.gather(table, 20)
    assert np.array_equal(K, quant.roundtrip(k))
    assert np.array_equal(V, quant.roundtrip(v))
    # unwritten slots read as NaN
    K2, _ = a.gather([4, 1], 32)
    assert np.isnan(K2[20:]).all()
    # the byte image of one block's K tiles: per head 16 * D codes + 16 fp16
    # scales, padded to whole 128-byte lines
    tile = arena.quant_tile_size(D)
    assert tile == 640 and arena.quant_tile_size(128) == 2176
    assert a.tile_bytes("k", 4).size == H * tile
    assert a.swap_out([4, 1]).size == 2 * 2 * H * tile
    # K codes of slot s at position kpos(s) (bits 2 and 3 exchanged), V codes
    # and both scale arrays in slot order, padding never written
    assert [int(x) for x in arena.kpos(np.arange(16))] == [0, 1, 2, 3, 8, 9, 10, 11,
                                                           4, 5, 6, 7, 12, 13, 14, 15]
    img_k, img_v = a.image("k")[4, 0], a.image("v")[4, 0]
    piece = img_k[:16 * D].reshape(D // 16, 16, 16)
    assert np.array_equal(piece[:, 8], a.kq[4, 0, :, 4].view(np.uint8))   # slot 4 at position 8
    assert np.array_equal(piece[:, 4], a.kq[4, 0, :, 8].view(np.uint8))   # slot 8 at position 4
    assert np.array_equal(img_v[:16 * D].reshape(D, 16), a.vq[4, 0].view(np.uint8))
    assert np.array_equal(img_k[16 * D:16 * D + 32].view(np.float16), a.ks[4, 0])
    assert (img_k[16 * D + 32:] == 0xFF).all() and (img_v[16 * D + 32:] == 0xFF).all()


@pytest.mark.parametrize("D", [32, 96, 128])
def test_int4_tile_image_layout(D):
    """INT4 arena image: K records per 16-dim piece at k4_record(slot) (the two
    keys a decode lane reads for MFMA u = 0, 1 adjacent), each byte holding dims
    i (low nibble) and 8 + i; V words of 4 bytes per (dim, key half) grouped by
    64 dims, byte i of half h holding slots 8h + i and 8h + 4 + i; codes as
    two's-complement nibbles; scales in slot order; padding to 128-byte lines."""
    rng = np.random.default_rng(6)
    H = 1
    a = arena.QuantArena(3, H, D, bits=4)
    k = _groups(rng, 16 * H, D).reshape(16, H, D)
    v = _groups(rng, 16 * H, D).reshape(16, H, D)
    a.write([2], 0, k, v)
    assert arena.quant_tile_size(32, 4) == 384 and arena.quant_tile_size(128, 4) == 1152
    rec = arena.k4_record(np.arange(16))
    assert sorted(rec.tolist()) == list(range(16))
    assert [int(x) for x in rec[[0, 4, 1, 5, 8, 12]]] == [0, 1, 2, 3, 8, 9]
    img_k, img_v = a.image("k")[2, 0], a.image("v")[2, 0]
    qk, _ = quant.encode(k, 4)                     # [16 slots][H][D]
    qv, _ = quant.encode(v, 4)
    for s in range(16):
        for p in range(D // 16):
            for i in range(8):
                byte = int(img_k[p * 128 + int(rec[s]) * 8 + i])
                lo, hi = byte & 15, byte >> 4
                assert lo == int(qk[s, 0, 16 * p + i]) & 15
                assert hi == int(qk[s, 0, 16 * p + 8 + i]) & 15
    # V: every code byte is used exactly once; group j of G dim blocks at 512 j
    offs = arena.v4_byte(np.arange(D)[:, None], np.arange(16)[None, :], D)
    assert np.array_equal(offs, arena.v4_byte(np.arange(D)[:, None], np.arange(16)[None, :] ^ 4, D))
    assert sorted(set(offs.ravel().tolist())) == list(range(8 * D))
    for d in range(D):
        j, G = d // 64, (4 if D - 64 * (d // 64) >= 64 else 2)
        for h in range(2):
            for i in range(4):
                at = 512 * j + 4 * ((16 * h + d % 16) * G + (d // 16) % 4) + i
                assert int(offs[d, 8 * h + i]) == at
                byte = int(img_v[at])
                assert byte & 15 == int(qv[8 * h + i, 0, d]) & 15
                assert byte >> 4 == int(qv[8 * h + 4 + i, 0, d]) & 15
    assert np.array_equal(img_k[8 * D:8 * D + 32].view(np.float16), a.ks[2, 0])
    assert (img_k[8 * D + 32:] == 0xFF).all()
    # unwritten blocks: all-ones bytes
    assert (a.image("k")[0] == 0xFF).all() and (a.image("v")[1] == 0xFF).all()
