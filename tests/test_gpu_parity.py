"""GPU parity: the HIP library against the CPU oracle (needs an MI355X).

Every case runs a seeded workload through libpkv (pool script on the library
pool, cache fills and the step's append through kv_append_rope, copy-on-write
through pkv_copy_blocks, then paged_attention_chunk / paged_attention_decode)
and through the oracle, and compares:
  * block tables, rotated queries and arena contents: bit for bit;
  * attention outputs: max |gpu - oracle| <= 2e-3 and mean <= 2e-4 (fp16
    inputs, fp32 accumulation; fp32 workloads share the bound).
Small workloads are compared element by element everywhere; the full-size
decode and chunk workloads are compared in full; the mixed and long-context
workloads on many sampled sequences and rows (their K/V regenerated and
rotated by the oracle for just those sequences, in worker processes), with
those sequences' arena blocks compared bit for bit.
"""
import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle_jobs  # noqa: E402
import paged_kv_chunked_amd as pkv  # noqa: E402
from oracle import rope as orope  # noqa: E402
from oracle import script as oscript  # noqa: E402
from paged_kv_chunked_amd import harness, workloads  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
MEAN_ABS = 2e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built")
    pkv.lib()


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


class Errors:
    """Output errors, in units of the workload's V scale (the outputs are linear
    in V, so their rounding errors scale with it)."""

    def __init__(self, scale=1.0):
        self.max = 0.0
        self.sum = 0.0
        self.n = 0
        self.scale = scale

    def add(self, got, exp):
        d = np.abs(np.asarray(got, np.float64) - exp) / self.scale
        assert np.isfinite(d).all(), "non-finite output"
        self.max = max(self.max, float(d.max()))
        self.sum += float(d.sum())
        self.n += d.size

    def check(self, name):
        mean = self.sum / max(self.n, 1)
        say(f"{name}: {self.n} outputs, max abs {self.max:.3e}, mean abs {mean:.3e}")
        assert self.max <= MAX_ABS, (name, self.max)
        assert mean <= MEAN_ABS, (name, mean)


def quant_image(a, which):
    """Byte image [N][Hkv][tile] of the oracle's quantized arena."""
    return a.image(which)


def run_case(w, full_arena=True, dec_sample=None, chunk_sample=None):
    """Runs workload w on the GPU and checks it against the oracle."""
    say(f"{w.name}: set-up (blocks={w.num_blocks}, step rows={len(w.step)})")
    dw = harness.DeviceWorkload(w)
    say(f"{w.name}: step")
    dw.step()
    torch.cuda.synchronize()
    say(f"{w.name}: oracle")
    st = oscript.run_script(w, materialize=full_arena)
    assert dw.copies == st.copies
    assert np.array_equal(dw.bt_host, oscript.block_table(w, st))
    q_rot = oscript.append_step(w, st)
    assert np.array_equal(bits(dw.q.cpu().numpy()), bits(q_rot)), "rotated q differs"
    if full_arena and w.kv_bits:
        assert np.array_equal(dw.k_arena.cpu().numpy(), quant_image(st.arena, "k")), "K arena differs"
        assert np.array_equal(dw.v_arena.cpu().numpy(), quant_image(st.arena, "v")), "V arena differs"
    elif full_arena:
        assert np.array_equal(bits(dw.k_arena.cpu().numpy()), bits(st.arena.k)), "K arena differs"
        assert np.array_equal(bits(dw.v_arena.cpu().numpy()), bits(st.arena.v)), "V arena differs"
    errs = Errors(w.v_scale)
    cu = dw.cu_host
    dec_rows = dw.dec_rows if dec_sample is None else dec_sample
    for r in dec_rows:
        s = w.step[r]
        if not full_arena and not w.kv_bits:  # the sampled sequence's arena blocks, bit for bit
            K, V = oscript.sequence_kv(w, st, r)
            L = s.start + 1
            tab = torch.tensor(dw.tables[s.seq][:-(-L // 16)], device=dw.device)
            kg = dw.k_arena.index_select(0, tab).cpu().numpy()
            vg = dw.v_arena.index_select(0, tab).cpu().numpy()
            kg = kg.transpose(0, 3, 1, 2, 4).reshape(-1, w.num_kv_heads, w.head_dim)[:L]
            vg = vg.transpose(0, 3, 1, 2).reshape(-1, w.num_kv_heads, w.head_dim)[:L]
            assert np.array_equal(bits(kg), bits(K)) and np.array_equal(bits(vg), bits(V))
        exp = oscript.attend_row(w, st, r, q_rot[cu[r]:cu[r + 1]], dw.scale)[0]
        errs.add(dw.dec_out[r - dw.dec_rows[0]].cpu().numpy(), exp)
    chunk_rows = dw.chunk_rows if chunk_sample is None else list(chunk_sample)
    for r in chunk_rows:
        s = w.step[r]
        rows = None
        if chunk_sample is not None:
            rng = np.random.default_rng(r)
            rows = np.unique(np.concatenate([[0, s.count - 1],
                                             rng.integers(0, s.count, size=chunk_sample[r])]))
        exp = oscript.attend_row(w, st, r, q_rot[cu[r]:cu[r + 1]], dw.scale, rows=rows)
        t0 = cu[r] - dw.chunk_tok0
        got = dw.chunk_out[t0:t0 + s.count].cpu().numpy()
        errs.add(got if rows is None else got[rows], exp)
    errs.check(w.name)
    return dw, st, q_rot


# ---------------------------------------------------------------------------
# small workloads: every element
# ---------------------------------------------------------------------------

def small_decode():
    lens = [1, 2, 15, 16, 17, 100, 255, 256, 257, 258, 511, 512, 513, 1000, 1600, 2049]
    return workloads.build("small_decode", 11, "f16", 32, 8, 128, 5.0e5,
                           [(L - 1, 1) for L in lens], max_blocks_per_seq=130)


def small_chunk():
    seqs = [(0, 1), (0, 33), (48, 16), (5, 70), (100, 129), (0, 200), (300, 64), (17, 5),
            (1000, 31), (64, 64)]
    return workloads.build("small_chunk", 12, "f16", 32, 8, 128, 5.0e5, seqs,
                           max_blocks_per_seq=80)


def split_prefix_one():
    """One 128-row chunk after a 6000-token prefix: 16 work units, so the call
    splits every tile's keys into 7 parts (one per 768 keys)."""
    return workloads.build("split_prefix_one", 14, "f16", 32, 8, 128, 5.0e5, [(6000, 128)],
                           max_blocks_per_seq=384)


def split_prefix_three():
    """Three short chunks with prefixes of 2000, 40 and 3500 tokens: 4 key parts,
    some of them holding no key of a row (or of a whole short item)."""
    return workloads.build("split_prefix_three", 15, "f16", 32, 8, 128, 5.0e5,
                           [(2000, 64), (40, 20), (3500, 100)], max_blocks_per_seq=226)


def small_mixed():
    return workloads.mixed_step(num_chunks=2, chunk=96, num_decodes=40, lo=1, hi=1200,
                                num_sharers=5, shared_prefix=256, parent_tokens=264)


def generic_shape(name, dtype, hq, hkv, d):
    seqs = [(0, 1), (40, 1), (299, 1), (0, 20), (37, 45)]
    return workloads.build(name, 13, dtype, hq, hkv, d, 1.0e4, seqs, max_blocks_per_seq=24)


def few_heads(name, hkv, lens, chunks=()):
    """The tuned shape (head dim 128, 4 query heads per KV head) with 2 or 4 KV
    heads: decode rows of the given contexts (and chunk rows (P, C))."""
    seqs = [(L - 1, 1) for L in lens] + list(chunks)
    return workloads.build(name, 17, "f16", 4 * hkv, hkv, 128, 5.0e5, seqs)


def i8(w):
    """The same workload over INT8 arenas (codes + fp16 scale per head vector)."""
    return dataclasses.replace(w, name=w.name + "_i8", kv_bits=8)


def i4(w):
    """The same workload over INT4 arenas (4-bit codes + fp16 scale per head vector)."""
    return dataclasses.replace(w, name=w.name + "_i4", kv_bits=4)


SMALL = {
    "tiny_f32": workloads.tiny,
    "small_decode": small_decode,
    "small_chunk": small_chunk,
    "small_mixed": small_mixed,
    "split_prefix_one": split_prefix_one,
    "split_prefix_three": split_prefix_three,
    "generic_f16_d64": lambda: generic_shape("generic_f16_d64", "f16", 8, 2, 64),
    "generic_f16_g2": lambda: generic_shape("generic_f16_g2", "f16", 8, 4, 128),
    "generic_f16_g8": lambda: generic_shape("generic_f16_g8", "f16", 16, 2, 128),
    "generic_f32_d128": lambda: generic_shape("generic_f32_d128", "f32", 8, 2, 128),
    "small_decode_i8": lambda: i8(small_decode()),
    "small_chunk_i8": lambda: i8(small_chunk()),
    "small_mixed_i8": lambda: i8(small_mixed()),
    "generic_i8_d64": lambda: i8(generic_shape("generic_i8_d64", "f16", 8, 2, 64)),
    "generic_i8_g2": lambda: i8(generic_shape("generic_i8_g2", "f16", 8, 4, 128)),
    "small_decode_i4": lambda: i4(small_decode()),
    "small_chunk_i4": lambda: i4(small_chunk()),
    "small_mixed_i4": lambda: i4(small_mixed()),
    "generic_i4_d64": lambda: i4(generic_shape("generic_i4_d64", "f16", 8, 2, 64)),
    "generic_i4_g2": lambda: i4(generic_shape("generic_i4_g2", "f16", 8, 4, 128)),
    # head dims that end in a short group: INT4 V words of 2 dim blocks, INT8 K
    # with an odd number of 16-dim pieces
    "generic_i4_d96": lambda: i4(generic_shape("generic_i4_d96", "f16", 8, 2, 96)),
    "generic_i8_d48": lambda: i8(generic_shape("generic_i8_d48", "f16", 8, 2, 48)),
    # V values up to ~4e4 (N(0, 1) x 2^13): the fp16 products of probability and
    # V scale must not overflow (INT4 scales reach 65504 / 7)
    "large_v_decode_i4": lambda: dataclasses.replace(i4(small_decode()), name="large_v_decode_i4",
                                                     v_scale=8192.0),
    "large_v_decode_i8": lambda: dataclasses.replace(i8(small_decode()), name="large_v_decode_i8",
                                                     v_scale=8192.0),
    "large_v_chunk": lambda: dataclasses.replace(small_chunk(), name="large_v_chunk",
                                                 v_scale=8192.0),
    # the quantized chunk kernel (dequantized into fp16 tiles in LDS)
    "large_v_chunk_i8": lambda: dataclasses.replace(i8(small_chunk()), name="large_v_chunk_i8",
                                                    v_scale=8192.0),
    "large_v_chunk_i4": lambda: dataclasses.replace(i4(small_chunk()), name="large_v_chunk_i4",
                                                    v_scale=8192.0),
    "split_prefix_one_i8": lambda: i8(split_prefix_one()),
    "split_prefix_three_i4": lambda: i4(split_prefix_three()),
    # the largest head dim the library accepts
    "generic_f16_d256": lambda: generic_shape("generic_f16_d256", "f16", 8, 2, 256),
    "generic_f32_d256": lambda: generic_shape("generic_f32_d256", "f32", 4, 2, 256),
    "generic_i4_d256": lambda: i4(generic_shape("generic_i4_d256", "f16", 8, 2, 256)),
    # fast paths with 2 or 4 KV heads (2- and 4-wave decode workgroups)
    "few_heads_hkv2": lambda: few_heads("few_heads_hkv2", 2, [1, 40, 383, 384, 385, 1000, 3001],
                                        chunks=[(37, 45)]),
    "few_heads_hkv4_wide": lambda: few_heads(
        "few_heads_hkv4_wide", 4,
        [int(x) for x in np.random.default_rng(5).integers(1, 4097, 40)]),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small(name):
    run_case(SMALL[name]())


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------

def test_decode_full():
    run_case(workloads.decode_batch())


def test_chunk_full():
    run_case(workloads.chunk_batch())


def test_chunk_full_i8():
    w = i8(workloads.chunk_batch())
    run_case(w, chunk_sample={r: 48 for r in w.chunk_rows()})


def test_chunk_full_i4():
    w = i4(workloads.chunk_batch())
    run_case(w, chunk_sample={r: 48 for r in w.chunk_rows()})


def test_tp8_shard_decode():
    """One GPU's share of the decode workload split by KV head over 8 GPUs
    (Hq 4 / Hkv 1): every output and the whole arena."""
    run_case(workloads.tp8_decode_batch())


def many_units(bits=0):
    """300 chunks of U[2, 130] rows after prefixes of 16 * U{0..24} tokens:
    ~3600 (row tile, KV head) units with rows among 7200 listed, so every
    persistent chunk workgroup computes a dozen or more units back to back
    (one-tile units included) and skips the empty ones."""
    rng = np.random.default_rng(16)
    rows = rng.integers(2, 130, size=300, endpoint=True)
    pre = 16 * rng.integers(0, 24, size=300, endpoint=True)
    w = workloads.build("many_units", 16, "f16", 32, 8, 128, 5.0e5,
                        [(int(p), int(c)) for p, c in zip(pre, rows)], max_blocks_per_seq=33)
    return dataclasses.replace(w, name=f"many_units_i{bits}", kv_bits=bits) if bits else w


@pytest.mark.parametrize("bits", [0, 8, 4])
def test_many_units(bits):
    """Every row of every chunk against the oracle when each workgroup walks
    many units (fp16, INT8 and INT4 arenas)."""
    w = many_units(bits)
    run_case(w, full_arena=False)


def test_tp8_shard_chunk():
    """One GPU's share of the chunk workload split by KV head over 8 GPUs
    (Hq 4 / Hkv 1; 64 row tiles, so the call splits keys into parts)."""
    run_case(workloads.tp8_chunk_batch())


@pytest.mark.parametrize("bits", [8, 4])
def test_tp8_shard_quant(bits):
    """The same shard shape over INT8 / INT4 arenas (decode and chunk)."""
    q = i8 if bits == 8 else i4
    run_case(q(workloads.tp8_decode_batch()))
    run_case(q(workloads.tp8_chunk_batch()))


def test_decode_full_i8():
    run_case(i8(workloads.decode_batch()))


def test_decode_full_i4():
    run_case(i4(workloads.decode_batch()))


# ---------------------------------------------------------------------------
# mixed and long-context workloads: many sampled rows, oracle in worker
# processes (symbolic oracle arena: a sequence's keys are regenerated when
# its rows are checked)
# ---------------------------------------------------------------------------

def edge_and_random_rows(count, n_random, seed):
    """Query rows of a chunk: the first and the last 64-row tile, plus
    ``n_random`` random rows."""
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(min(64, count)), np.arange(max(0, count - 64), count),
                           rng.integers(0, count, size=n_random)])
    return np.unique(rows)


def run_sampled(w, dec_rows, chunk_rows, block_rows, chunk_jobs=8):
    """Runs workload w on the GPU (pool script, fills, step append, chunk and
    decode calls) and checks against the oracle:
      * block tables, copy-on-write copies and every rotated query, bit for bit;
      * the arena blocks of the sequences of ``block_rows``, bit for bit
        (digests of the GPU's tiles against the oracle's images);
      * the outputs of decode rows ``dec_rows`` and of the query rows
        ``chunk_rows[r]`` of chunk row r, within the tolerance."""
    say(f"{w.name}: set-up (blocks={w.num_blocks}, step rows={len(w.step)})")
    dw = harness.DeviceWorkload(w)
    say(f"{w.name}: step")
    dw.step()
    torch.cuda.synchronize()
    say(f"{w.name}: oracle script")
    st = oscript.run_script(w, materialize=False)
    assert dw.copies == st.copies
    assert np.array_equal(dw.bt_host, oscript.block_table(w, st))
    q_rot = oscript.append_step(w, st)
    assert np.array_equal(bits(dw.q.cpu().numpy()), bits(q_rot)), "rotated q differs"
    block_rows = set(block_rows)
    jobs = [(r, None, r in block_rows) for r in dec_rows]
    for r, rows in chunk_rows.items():
        for i, part in enumerate(np.array_split(np.asarray(rows), chunk_jobs)):
            if part.size:
                jobs.append((r, part, i == 0 and r in block_rows))
    say(f"{w.name}: oracle, {len(jobs)} jobs ({len(dec_rows)} decode rows, "
        f"{sum(len(v) for v in chunk_rows.values())} chunk rows, {len(block_rows)} sequences' blocks)")
    results = oracle_jobs.run(w, st, q_rot, dw.cu_host, jobs, dw.scale)
    errs = Errors(w.v_scale)
    cu = dw.cu_host
    for r, rows, exp, dk, dv in results:
        s = w.step[r]
        if dk is not None:
            nb = -(-(s.start + s.count) // w.block_size)
            tab = torch.tensor(dw.tables[s.seq][:nb], device=dw.device, dtype=torch.int64)
            gk = dw.k_arena.index_select(0, tab).cpu().numpy()
            gv = dw.v_arena.index_select(0, tab).cpu().numpy()
            assert oracle_jobs.digest(gk) == dk, ("K blocks differ", r)
            assert oracle_jobs.digest(gv) == dv, ("V blocks differ", r)
        if s.count == 1:
            got = dw.dec_out[r - dw.dec_rows[0]].cpu().numpy()[None]
        else:
            t0 = cu[r] - dw.chunk_tok0
            got = dw.chunk_out[t0:t0 + s.count].cpu().numpy()[rows]
        errs.add(got, exp)
    errs.check(w.name)
    return dw


def mixed_rows(w, total=128, seed=0):
    """Decode rows of the mixed step to check, ``total`` of them: every row
    sharing the prefix, the 32 longest contexts (their batch's split partials
    exceed 64 MiB, so the combine takes its 2-split prefetch form), and random
    others."""
    dec = w.decode_rows()
    sharers = [op[1] for op in w.script if op[0] == "fork"]
    longest = sorted(dec, key=lambda r: -w.step[r].start)[:32]
    chosen = set(sharers) | set(longest)
    rng = np.random.default_rng(seed)
    rest = [r for r in dec if r not in chosen]
    extra = rng.choice(rest, size=max(total - len(chosen), 0), replace=False).tolist()
    return sorted(chosen | set(extra))


def test_mixed_full_sampled():
    """The 2048-token-budget step (4 chunks of 256 + 1024 decodes, 16 sharing
    a 1024-token prefix) through the separate chunk and decode calls: 128
    decode rows and every chunk row against the oracle, and every checked
    sequence's arena blocks bit for bit."""
    w = workloads.mixed_step()
    dec = mixed_rows(w)
    assert len(dec) >= 128
    chunks = {r: np.arange(w.step[r].count) for r in w.chunk_rows()}
    run_sampled(w, dec, chunks, block_rows=dec + list(chunks), chunk_jobs=2)


def _long_rows(w):
    r = w.chunk_rows()[0]
    return w.decode_rows(), {r: edge_and_random_rows(w.step[r].count, 400, seed=r)}


def test_long_full_sampled():
    """The long workload: 32 decodes at context 32768 and one 4096-row chunk
    after 28,672 cached tokens, 1% of key vectors x8 (fp16 arena): every
    decode row, the first and last 64-row tiles of the chunk plus 400 random
    rows, and every sequence's arena blocks bit for bit."""
    w = workloads.long_context()
    dec, chunks = _long_rows(w)
    run_sampled(w, dec, chunks, block_rows=dec + list(chunks))


def test_long_full_sampled_i8():
    """The long workload over an INT8 arena (same rows and blocks checked)."""
    w = i8(workloads.long_context())
    dec, chunks = _long_rows(w)
    run_sampled(w, dec, chunks, block_rows=dec[:4] + list(chunks))


def test_long_full_sampled_i4():
    """The long workload over an INT4 arena (same rows and blocks checked)."""
    w = i4(workloads.long_context())
    dec, chunks = _long_rows(w)
    run_sampled(w, dec, chunks, block_rows=dec[:4] + list(chunks))


# ---------------------------------------------------------------------------
# invariants on the GPU path
# ---------------------------------------------------------------------------

def _same_data_other_blocks(seed_perm):
    seqs = [(L - 1, 1) for L in (300, 1000, 17, 2500)] + [(77, 150), (0, 64)]
    return workloads.build("perm", 21, "f16", 32, 8, 128, 5.0e5, seqs, slack=1.5,
                           max_blocks_per_seq=160,
                           shuffle_rng=np.random.default_rng(seed_perm))


def test_block_permutation_invariance_bitwise():
    outs = []
    for sp in (1, 2):
        w = _same_data_other_blocks(sp)
        say(f"permutation {sp}")
        dw = harness.DeviceWorkload(w)
        dw.step()
        torch.cuda.synchronize()
        outs.append((dw.bt_host.copy(), dw.dec_out.cpu().numpy(), dw.chunk_out.cpu().numpy()))
    assert not np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(bits(outs[0][1]), bits(outs[1][1]))
    assert np.array_equal(bits(outs[0][2]), bits(outs[1][2]))


def test_batch_invariance_bitwise():
    w = workloads.decode_batch(num_seqs=16, lo=1, hi=3000)
    say("batch invariance")
    dw = harness.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    full = dw.dec_out.cpu().numpy()
    for r in (0, 5, 15):
        out = torch.empty((1, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dw.device)
        L = int(dw.dec_lens_host[r])
        ws_n = pkv.paged_attention_decode_workspace_bytes(dw.g, 1, L)
        ws = torch.zeros(max(ws_n, 4) // 4, dtype=torch.float32, device=dw.device) if ws_n else None
        pkv.paged_attention_decode(dw.g, out, dw.dec_q[r:r + 1], dw.k_arena, dw.v_arena,
                                   dw.dec_bt[r:r + 1], dw.dec_lens[r:r + 1], L, dw.scale, ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out.cpu().numpy()[0]), bits(full[r]))


def test_single_key_returns_v_exactly():
    w = workloads.build("one_key", 31, "f16", 32, 8, 128, 5.0e5, [(0, 1), (0, 1)],
                        max_blocks_per_seq=2)
    dw = harness.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    _, _, v = w.draw_step_packed()
    out = dw.dec_out.cpu().numpy()
    for b in range(2):
        for h in range(32):
            assert np.array_equal(out[b, h], v[b, h // 4].astype(np.float32))


def test_decode_matches_last_chunk_row():
    w = workloads.build("last_row", 41, "f16", 32, 8, 128, 5.0e5, [(700, 100)],
                        max_blocks_per_seq=60)
    dw = harness.DeviceWorkload(w)
    dw.step()
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dw.device)
    lens = torch.tensor([800], dtype=torch.int32, device=dw.device)
    ws_n = pkv.paged_attention_decode_workspace_bytes(dw.g, 1, 800)
    ws = torch.zeros(ws_n // 4, dtype=torch.float32, device=dw.device)
    pkv.paged_attention_decode(dw.g, out, dw.chunk_q[99:100], dw.k_arena, dw.v_arena,
                               dw.chunk_bt, lens, 800, dw.scale, ws)
    torch.cuda.synchronize()
    d = np.abs(out.cpu().numpy()[0] - dw.chunk_out[99].cpu().numpy())
    assert d.max() <= MAX_ABS


def test_copy_blocks_bitwise_and_skips_bad_pairs():
    g = pkv.geom(8, 2, 8, 64)
    k = torch.randn(8, 2, 8, 16, 8, device="cuda").half()
    v = torch.randn(8, 2, 64, 16, device="cuda").half()
    k0, v0 = k.clone(), v.clone()
    pairs = torch.tensor([[1, 5], [2, 6], [3, 99], [-1, 0]], dtype=torch.int32, device="cuda")
    pkv.pkv_copy_blocks(g, k, v, pairs)
    torch.cuda.synchronize()
    exp_k, exp_v = k0.clone(), v0.clone()
    exp_k[5], exp_v[5] = k0[1], v0[1]
    exp_k[6], exp_v[6] = k0[2], v0[2]
    assert torch.equal(k.view(torch.int16), exp_k.view(torch.int16))
    assert torch.equal(v.view(torch.int16), exp_v.view(torch.int16))


def test_empty_and_degenerate_batches():
    g = pkv.geom(4, 8, 32, 128)
    dev = "cuda"
    k_ar = torch.zeros(4, 8, 16, 16, 8, dtype=torch.float16, device=dev)
    v_ar = torch.zeros(4, 8, 128, 16, dtype=torch.float16, device=dev)
    bt = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device=dev)
    # a chunk batch with an empty sequence in the middle
    cu = torch.tensor([0, 3, 3, 5], dtype=torch.int32, device=dev)
    starts = torch.tensor([0, 7, 20], dtype=torch.int32, device=dev)
    bt3 = torch.tensor([[0, 1], [2, 3], [1, 0]], dtype=torch.int32, device=dev)
    q = torch.randn(5, 32, 128, device=dev).half()
    out = torch.full((5, 32, 128), float("nan"), device=dev)
    pkv.paged_attention_chunk(g, out, q, k_ar, v_ar, bt3, cu, starts, 3, 25, 0.1)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    # decode rows of length 0 give zeros
    lens = torch.tensor([0, 5], dtype=torch.int32, device=dev)
    outd = torch.full((2, 32, 128), float("nan"), device=dev)
    pkv.paged_attention_decode(g, outd, q[:2].contiguous(), k_ar, v_ar, bt, lens, 32, 0.1, None)
    torch.cuda.synchronize()
    assert torch.equal(outd[0], torch.zeros_like(outd[0])) and torch.isfinite(outd[1]).all()
