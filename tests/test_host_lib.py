"""Host-side tests of libpkv (CPU only, no GPU calls).

  * the library loads and exports every function include/pkv.h declares;
  * the library pool equals the oracle pool bit for bit (ids handed out,
    copy-on-write decisions, free-list order) on random operation sequences
    and on every workload's pool script;
  * the library's RoPE table equals the oracle's bit for bit;
  * the library's fp64 -> fp16 rounding equals numpy's (itself pinned to exact
    rational rounding in test_oracle_rope.py);
  * argument validation of every entry point (errors return before anything
    is launched, so these calls are safe without a GPU).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_chunked_amd as pkv
from oracle import pool as opool
from oracle import rope as orope
from oracle import script as oscript
from paged_kv_chunked_amd import harness, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        pytest.skip("libpkv.so not built")
    return pkv.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert pkv.pkv_abi_version() == 1


def test_library_matches_its_sources(lib):
    """The library embeds the hash of the sources and flags it was built from;
    the binding refuses a library whose hash differs from the sources beside it."""
    from paged_kv_chunked_amd import build as pkv_build
    h = pkv.pkv_source_hash()
    assert len(h) == 64 and all(c in "0123456789abcdef" for c in h)
    assert h == pkv_build.source_hash()


def test_rope_table_bitwise_equals_oracle(lib):
    for theta, D, max_pos in [(1.0e4, 64, 700), (5.0e5, 128, 9000)]:
        ours = np.empty((max_pos, D // 2, 2), np.float64)
        pkv.pkv_rope_table_host(ours, theta, D, max_pos)
        cos, sin = orope.cos_sin_table(theta, D, max_pos)
        assert np.array_equal(ours[..., 0].view(np.uint64), cos.view(np.uint64))
        assert np.array_equal(ours[..., 1].view(np.uint64), sin.view(np.uint64))
    assert pkv.pkv_rope_table_bytes(128, 10) == 10 * 64 * 16


def test_f64_to_f16_matches_numpy(lib):
    rng = np.random.default_rng(0)
    special = np.array([0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, np.inf, -np.inf,
                        2.0 ** -24, 2.0 ** -25, 2.0 ** -25 + 2.0 ** -50, 3 * 2.0 ** -25,
                        2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 2.0 ** -1030, 5e-324,
                        1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -40])
    mant = rng.integers(0, 2 ** 11, size=20000)
    ties = (1.0 + (2 * mant + 1) * 2.0 ** -12) * 2.0 ** rng.integers(-26, 16, size=20000)
    near = ties * (1 + rng.choice([-1, 1], size=20000) * 2.0 ** -45)
    bits = rng.integers(0, 2 ** 64 - 1, size=20000, dtype=np.uint64).view(np.float64)
    bits = bits[np.isfinite(bits)]
    x = np.concatenate([special, -special, ties, -ties, near, bits,
                        rng.standard_normal(100000) * 4, rng.standard_normal(20000) * 1e-5])
    ours = np.empty(x.size, np.uint16)
    pkv.pkv_f64_to_f16_host(x, ours)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = np.array([np.nan])
    o = np.empty(1, np.uint16)
    pkv.pkv_f64_to_f16_host(nan, o)
    assert (o[0] & 0x7C00) == 0x7C00 and (o[0] & 0x3FF) != 0


# ---------------------------------------------------------------------------
# pool
# ---------------------------------------------------------------------------

def test_pool_random_ops_match_oracle(lib):
    rng = np.random.default_rng(3)
    for trial in range(5):
        N = int(rng.integers(1, 40))
        a, b = pkv.Pool(N), opool.Pool(N)
        held = []
        for _ in range(3000):
            r = rng.random()
            if r < 0.35:
                if b.num_free:
                    x = b.alloc()
                    assert a.alloc() == x
                    held.append(x)
                else:
                    with pytest.raises(pkv.PkvError) as e:
                        a.alloc()
                    assert e.value.code == 6
            elif r < 0.5 and held:
                x = held[int(rng.integers(len(held)))]
                a.incref(x)
                b.incref(x)
                held.append(x)
            elif r < 0.65 and held:
                i = int(rng.integers(len(held)))
                x = held[i]
                if b.refcount[x] > 1 and not b.num_free:
                    continue
                nb, cb = b.cow(x)
                na, ca = a.cow(x)
                assert (na, ca) == (nb, cb)
                held[i] = nb
            elif held:
                x = held.pop(int(rng.integers(len(held))))
                a.decref(x)
                b.decref(x)
            assert a.num_free == b.num_free
            assert list(a.free_list()) == b.free
        for x in range(N):
            assert a.refcount(x) == b.refcount.get(x, 0)


def test_pool_errors(lib):
    p = pkv.Pool(2)
    with pytest.raises(pkv.PkvError) as e:
        p.decref(0)
    assert e.value.code == 7
    with pytest.raises(pkv.PkvError) as e:
        p.incref(5)
    assert e.value.code == 4
    with pytest.raises(pkv.PkvError) as e:
        p.alloc_n(3)
    assert e.value.code == 6 and p.num_free == 2      # all or nothing
    x = p.alloc()
    assert p.cow(x) == (x, False)
    assert lib.pkv_pool_create(0) is None


@pytest.mark.parametrize("make", [
    workloads.tiny,
    lambda: workloads.decode_batch(num_seqs=9, lo=1, hi=700),
    lambda: workloads.chunk_batch(num_seqs=3, chunk=100, max_prefix_blocks=20),
    lambda: workloads.mixed_step(num_chunks=2, chunk=40, num_decodes=30, lo=20, hi=600,
                                 num_sharers=4, shared_prefix=64, parent_tokens=72),
    workloads.decode_batch, workloads.chunk_batch, workloads.mixed_step,
])
def test_workload_tables_match_oracle(lib, make):
    w = make()
    tables = {s: [] for s in range(w.num_pool_seqs)}
    p = pkv.Pool(w.num_blocks)
    copies = harness.run_pool_script(w, p, tables)
    st = oscript.run_script(w, materialize=False)
    assert tables == st.tables
    assert copies == st.copies
    assert list(p.free_list()) == st.pool.free


def test_validate_tables(lib):
    g = pkv.geom(10, 2, 4, 64)
    bt = np.array([[3, 4, -1], [9, -1, -1]], np.int32)
    pkv.pkv_validate_tables(g, bt, np.array([20, 16], np.int32))
    for lens in ([20, 17], [49, 1], [-1, 1]):
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_validate_tables(g, bt, np.array(lens, np.int32))
        assert e.value.code == 4
    bad = bt.copy()
    bad[1, 0] = 10
    with pytest.raises(pkv.PkvError):
        pkv.pkv_validate_tables(g, bad, np.array([20, 16], np.int32))


# ---------------------------------------------------------------------------
# argument validation of the device entry points (nothing is launched)
# ---------------------------------------------------------------------------

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _geom(**kw):
    g = dict(num_blocks=64, block_size=16, num_kv_heads=8, num_q_heads=32, head_dim=128, dtype=0)
    g.update(kw)
    return pkv.Geom(**g)


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=32), 2), (dict(num_q_heads=30), 2), (dict(head_dim=130 * 2), 2),
    (dict(head_dim=3), 2), (dict(head_dim=12), 2), (dict(head_dim=6, dtype=1), 2),
    (dict(num_blocks=0), 2), (dict(dtype=7), 3), (dict(num_kv_heads=0), 2),
    (dict(head_dim=40, dtype=2), 2), (dict(head_dim=48, dtype=3), 2),
])
def test_bad_geometry_rejected(lib, kw, code):
    g = _geom(**kw)
    r = lib.kv_append_rope(ctypes.byref(g), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                           FAKE, 1, 1, FAKE, 100, None)
    assert r == code
    r = lib.paged_attention_decode(ctypes.byref(g), FAKE, 1, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1,
                                   64, 0.1, FAKE, 1 << 20, None)
    assert r == code
    r = lib.paged_attention_chunk(ctypes.byref(g), FAKE, 1, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE,
                                  1, 16, 16, 64, 0.1, None, 0, None)
    assert r == code
    assert lib.pkv_copy_blocks(ctypes.byref(g), FAKE, FAKE, FAKE, 1, None) == code


def test_entry_point_errors(lib):
    g = _geom()
    gp = ctypes.byref(g)
    # nulls
    assert lib.kv_append_rope(None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 1,
                              1, FAKE, 100, None) == 1
    assert lib.kv_append_rope(gp, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 1, 1,
                              FAKE, 100, None) == 1
    assert lib.paged_attention_decode(gp, None, 1, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 64, 0.1,
                                      FAKE, 1 << 20, None) == 1
    # empty batches are a no-op (no launch)
    assert lib.kv_append_rope(gp, None, None, None, None, None, None, None, 4, None, None, 0, 0,
                              None, 100, None) == 0
    assert lib.paged_attention_decode(gp, None, 1, None, None, None, None, 4, None, 0, 64, 0.1,
                                      None, 0, None) == 0
    assert lib.paged_attention_chunk(gp, None, 1, None, None, None, None, 4, None, None, 0, 0,
                                     16, 64, 0.1, None, 0, None) == 0
    assert lib.pkv_copy_blocks(gp, None, None, None, 0, None) == 0
    # dtype of the output
    assert lib.paged_attention_decode(gp, FAKE, 0, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 64, 0.1,
                                      FAKE, 1 << 20, None) == 3
    # context longer than the block table can hold
    assert lib.paged_attention_decode(gp, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 1, 65, 0.1,
                                      FAKE, 1 << 20, None) == 4
    assert lib.paged_attention_chunk(gp, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 1, 16,
                                     16, 65, 0.1, None, 0, None) == 4
    assert lib.paged_attention_chunk(gp, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 1, 16,
                                     32, 16, 0.1, None, 0, None) == 4
    # workspace
    need = pkv.paged_attention_decode_workspace_bytes(g, 3, 1000)
    parts = 3 * 32 * -(-1000 // 384)                 # sequences x heads x 384-token splits
    assert need == -(-parts * 128 * 4 // 256) * 256 + parts * 2 * 4
    assert pkv.paged_attention_decode_workspace_bytes(g, 3, 384) == 0   # one split: no partials
    assert lib.paged_attention_decode(gp, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 3, 1000,
                                      0.1, FAKE, need - 1, None) == 5
    assert lib.paged_attention_decode(gp, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 3, 1000,
                                      0.1, None, need, None) == 5
    # the allocation-free decode: batches whose partials exceed its static
    # scratch are refused before anything is launched (32 MiB: 64 sequences of
    # 32 heads hold up to 31 splits, i.e. contexts of 11,904 tokens)
    assert pkv.paged_attention_decode_workspace_bytes(g, 64, 31 * 384) <= 32 << 20
    assert pkv.paged_attention_decode_workspace_bytes(g, 64, 32 * 384) > 32 << 20
    assert lib.paged_attention_decode_noalloc(gp, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 800, FAKE, 64,
                                              32 * 384, 0.1, None) == 5
    assert lib.paged_attention_decode_noalloc(gp, None, 1, FAKE, FAKE, FAKE, FAKE, 800, FAKE, 64,
                                              384, 0.1, None) == 1
    assert lib.paged_attention_decode_noalloc(gp, None, 1, None, None, None, None, 4, None, 0,
                                              64, 0.1, None) == 0
    # the fused append + decode: argument checks before any launch
    A = ctypes.c_void_p(0x100000)
    B = ctypes.c_void_p(0x100000 + 3 * 32 * 128 * 2)          # right after A's 3 rows of q
    dec_app = lambda *a: lib.paged_attention_decode_append(gp, *a)
    assert dec_app(FAKE, 1, A, None, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 3, 1000, 0.1,
                   FAKE, 4096, FAKE, need, None) == 1          # q_out missing
    assert dec_app(FAKE, 1, A, ctypes.c_void_p(0x100000 + 64), FAKE, FAKE, FAKE, FAKE, FAKE, 64,
                   FAKE, 3, 1000, 0.1, FAKE, 4096, FAKE, need, None) == 4   # q_out overlaps q
    assert dec_app(FAKE, 1, A, B, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 3, 1000, 0.1,
                   FAKE, 0, FAKE, need, None) == 4             # no RoPE positions
    assert dec_app(FAKE, 1, A, B, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 3, 1000, 0.1,
                   FAKE, 4096, FAKE, need - 1, None) == 5      # workspace too small
    assert lib.paged_attention_decode_append(ctypes.byref(_geom(dtype=1)), FAKE, 1, A, B, FAKE,
                                             FAKE, FAKE, FAKE, FAKE, 64, FAKE, 3, 1000, 0.1,
                                             FAKE, 4096, FAKE, need, None) == 3   # fp32 arena
    assert lib.paged_attention_decode_append(ctypes.byref(_geom(dtype=2, num_q_heads=16)), FAKE,
                                             1, A, B, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 3,
                                             1000, 0.1, FAKE, 4096, FAKE, need,
                                             None) == 2        # INT8, group 2: not the fast path
    assert dec_app(None, 1, None, None, None, None, None, None, None, 4, None, 0, 64, 0.1,
                   None, 1, None, 0, None) == 0                # empty batch
    # chunk: the schedule, one int32 per (sequence, 64-row tile)
    need = pkv.paged_attention_chunk_workspace_bytes(g, 2, 100, 500)
    assert need == 2 * 2 * 4
    assert lib.paged_attention_chunk(gp, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, 2, 100,
                                     64, 500, 0.1, FAKE, need - 1, None) == 5
    assert lib.paged_attention_chunk(gp, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, 2, 100,
                                     64, 500, 0.1, None, need, None) == 5
    g32 = _geom(dtype=1)   # fp32 storage runs the generic kernel: no schedule
    assert pkv.paged_attention_chunk_workspace_bytes(g32, 2, 100, 500) == 0
    # the chunk call's two halves take its checks (the plan reads no q, out,
    # arena or block table)
    plan = lambda *a: lib.paged_attention_chunk_plan(gp, *a)
    assert plan(64, None, FAKE, 2, 100, 64, 500, FAKE, need, None) == 1     # cu_q_lens
    assert plan(64, FAKE, None, 2, 100, 64, 500, FAKE, need, None) == 1     # chunk_start
    assert plan(64, FAKE, FAKE, 2, 100, 64, 4000, FAKE, need, None) == 4    # context > table
    assert plan(64, FAKE, FAKE, 2, 100, 600, 500, FAKE, need, None) == 4    # rows > context
    assert plan(64, FAKE, FAKE, 2, 100, 64, 500, FAKE, need - 1, None) == 5
    assert plan(64, FAKE, FAKE, -1, 100, 64, 500, FAKE, need, None) == 4
    assert plan(64, None, None, 0, 0, 64, 500, None, 0, None) == 0          # empty batch
    assert lib.paged_attention_chunk_plan(None, 64, FAKE, FAKE, 2, 100, 64, 500, FAKE, need,
                                          None) == 1
    run = lambda *a: lib.paged_attention_chunk_run(gp, *a)
    assert run(FAKE, 0, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, 2, 100, 64, 500, 0.1, FAKE,
               need, None) == 3                                            # output dtype
    assert run(FAKE, 1, FAKE, FAKE, FAKE, None, 64, FAKE, FAKE, 2, 100, 64, 500, 0.1, FAKE,
               need, None) == 1                                            # block table
    assert run(FAKE, 1, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, 2, 100, 64, 500, 0.1, None,
               need, None) == 5
    assert run(None, 1, None, None, None, None, 4, None, None, 0, 0, 16, 64, 0.1, None, 0,
               None) == 0
    assert lib.pkv_status_string(5) == b"workspace missing or too small"


def test_chunk_key_range_parts(lib):
    """A chunk call with fewer than 512 (64-row tile, KV head) units splits each
    tile's keys into ceil(512 / units) parts, at most 8 and at most one per 768
    keys of the longest context; the workspace then holds the parts' partials."""
    g = _geom()   # Hq 32, Hkv 8, head_dim 128, fp16: the tuned path
    parts = lambda T, ctx, geom=g: pkv.paged_attention_chunk_parts(geom, 4, T, ctx)
    assert parts(4096, 4096) == 1           # 64 tiles x 8 heads = 512 units
    assert parts(1024, 8192) == 4           # 128 units
    assert parts(64, 32768) == 8            # 8 units: capped at 8
    assert parts(64, 1600) == 2             # at least 768 keys per part
    assert parts(64, 1500) == 1
    assert parts(256, 3632) == 4            # 64 units (one KV head)
    assert parts(100, 500) == 1             # too short to split
    assert parts(1024, 8192, _geom(dtype=1)) == 1     # generic path
    # workspace of a split call: schedule, then o [parts][T][Hq][D] and (m, l)
    rows = 4 * 1024 * 32
    assert pkv.paged_attention_chunk_workspace_bytes(g, 4, 1024, 8192) == \
        256 + rows * 128 * 4 + rows * 2 * 4
    n = ctypes.c_int32()
    gp = ctypes.byref(g)
    assert lib.paged_attention_chunk_parts(gp, 4, 1024, 8192, None) == 1
    assert lib.paged_attention_chunk_parts(gp, 4, -1, 8192, ctypes.byref(n)) == 4
    assert lib.paged_attention_chunk_parts(gp, 4, 1024, 8192, ctypes.byref(n)) == 0 and n.value == 4


@pytest.mark.parametrize("dtype", [2, 3])
def test_quantized_arenas_take_the_tuned_chunk_and_mixed_paths(lib, dtype):
    """INT8 / INT4 arenas at head_dim 128 and 4 query heads per KV head run the
    tuned chunk and mixed kernels: the same key-range parts, schedule and
    partials as fp16 (the partials are fp32 either way); other shapes of the
    same storage keep the generic path (no workspace, never split)."""
    g16, gq = _geom(), _geom(dtype=dtype)
    for T, ctx in ((4096, 4096), (1024, 8192), (64, 32768), (64, 1500), (100, 500)):
        assert pkv.paged_attention_chunk_parts(gq, 4, T, ctx) == \
            pkv.paged_attention_chunk_parts(g16, 4, T, ctx)
        assert pkv.paged_attention_chunk_workspace_bytes(gq, 4, T, ctx) == \
            pkv.paged_attention_chunk_workspace_bytes(g16, 4, T, ctx)
        assert pkv.paged_attention_mixed_workspace_bytes(gq, 4, T, ctx) == \
            pkv.paged_attention_mixed_workspace_bytes(g16, 4, T, ctx) > 0
    gen = _geom(dtype=dtype, num_q_heads=16)   # group 2: generic kernel
    assert pkv.paged_attention_chunk_parts(gen, 4, 64, 32768) == 1
    assert pkv.paged_attention_chunk_workspace_bytes(gen, 4, 64, 32768) == 0
    assert pkv.paged_attention_mixed_workspace_bytes(gen, 4, 64, 32768) == 0


def test_pool_admission_matches_oracle(lib):
    from oracle import pool as opool
    rng = np.random.default_rng(11)
    for _ in range(300):
        N = int(rng.integers(1, 50))
        p = pkv.Pool(N)
        taken = int(rng.integers(0, N + 1))
        for _ in range(taken):
            p.alloc()
        ev, res, need = (int(x) for x in rng.integers(0, 30, size=3))
        assert p.can_admit(ev, res, need) == opool.can_admit(N - taken, ev, res, need)
    with pytest.raises(pkv.PkvError):
        pkv.Pool(4).can_admit(-1, 0, 0)


def test_swap_entry_point_errors(lib):
    g = _geom()
    gp = ctypes.byref(g)
    tile = 8 * 16 * 128 * 2
    assert pkv.pkv_swap_bytes(g, 3) == 3 * 2 * tile
    # n == 0 is a no-op; nulls, a short or misaligned buffer are rejected before any launch
    assert lib.pkv_swap_out(gp, None, None, None, 0, None, 0, None) == 0
    assert lib.pkv_swap_out(gp, FAKE, FAKE, None, 2, FAKE, 2 * 2 * tile, None) == 1
    assert lib.pkv_swap_in(gp, FAKE, FAKE, FAKE, 2, FAKE, 2 * 2 * tile - 1, None) == 5
    assert lib.pkv_swap_in(gp, FAKE, FAKE, FAKE, 2, ctypes.c_void_p(0x1008), 2 * 2 * tile, None) == 4
    assert lib.pkv_swap_out(gp, FAKE, FAKE, FAKE, -1, FAKE, 0, None) == 4


def test_stream_read_helper_errors(lib):
    # the measurement helper rejects nulls, sizes not a multiple of 16 and a
    # misaligned source before any launch
    assert lib.pkv_stream_read(None, 16, FAKE, None) == 1
    assert lib.pkv_stream_read(FAKE, 16, None, None) == 1
    assert lib.pkv_stream_read(FAKE, 24, FAKE, None) == 4
    assert lib.pkv_stream_read(ctypes.c_void_p(0x1008), 16, FAKE, None) == 4


def test_mixed_entry_point_errors(lib):
    g = _geom()
    gp = ctypes.byref(g)
    args = lambda out, dt, ws, wsb, **kw: (gp, out, dt, FAKE, FAKE, FAKE, FAKE, kw.get("mb", 64),
                                           FAKE, FAKE, kw.get("S", 2), kw.get("T", 100),
                                           kw.get("mq", 64), kw.get("mc", 500), 0.1, ws, wsb, None)
    # empty batches are a no-op; nulls, the output dtype, a context longer than
    # the table and a short workspace are rejected before any launch
    assert lib.paged_attention_mixed(gp, None, 1, None, None, None, None, 4, None, None, 0, 0, 16,
                                     64, 0.1, None, 0, None) == 0
    assert lib.paged_attention_mixed(*args(None, 1, FAKE, 1 << 30)) == 1
    assert lib.paged_attention_mixed(*args(FAKE, 0, FAKE, 1 << 30)) == 3
    assert lib.paged_attention_mixed(*args(FAKE, 1, FAKE, 1 << 30, mc=64 * 16 + 1)) == 4
    assert lib.paged_attention_mixed(*args(FAKE, 1, FAKE, 1 << 30, mq=501)) == 4
    need = pkv.paged_attention_mixed_workspace_bytes(g, 2, 100, 500)
    # schedule (4 header ints + 2 x 2 row tiles + 2 x 2 splits, 256-aligned) +
    # the decode partials of 2 sequences x 2 splits
    parts = 2 * 32 * 2
    assert need == 256 + (-(-parts * 128 * 4 // 256) * 256 + parts * 2 * 4)
    assert lib.paged_attention_mixed(*args(FAKE, 1, FAKE, need - 1)) == 5
    assert lib.paged_attention_mixed(*args(FAKE, 1, None, need)) == 5
    # one split per context: the schedule only
    assert pkv.paged_attention_mixed_workspace_bytes(g, 2, 100, 384) == 256
    # fp32 storage runs the generic kernel: no workspace
    assert pkv.paged_attention_mixed_workspace_bytes(_geom(dtype=1), 2, 100, 500) == 0


def test_decode_shared_entry_point_errors(lib):
    g = _geom()
    gp = ctypes.byref(g)
    need = pkv.paged_attention_decode_workspace_bytes(g, 3, 1000)

    def call(out=FAKE, dt=1, gs=FAKE, rs=FAKE, ng=1, mskip=2, mgs=3, ws=FAKE, wsb=None, mc=1000):
        return lib.paged_attention_decode_shared(gp, out, dt, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 3,
                                                 mc, 0.1, gs, rs, ng, mskip, mgs, ws,
                                                 need if wsb is None else wsb, None)
    assert call(out=None) == 1
    assert call(gs=None) == 1 and call(rs=None) == 1
    assert call(dt=0) == 3
    assert call(ng=-1) == 4 and call(mskip=-1) == 4 and call(mgs=-1) == 4
    assert call(mc=64 * 16 + 1) == 4
    assert call(wsb=need - 1) == 5 and call(ws=None) == 5


@pytest.mark.parametrize("dtype,tile", [(0, 16 * 128 * 2), (2, 2176), (3, 1152)])
def test_swap_bytes_per_storage(lib, dtype, tile):
    """Swap buffers hold whole tiles: fp16 4 KiB, INT8 and INT4 tiles padded
    to 128-byte lines (codes + 16 scales)."""
    g = _geom(dtype=dtype)
    assert pkv.pkv_swap_bytes(g, 5) == 5 * 2 * 8 * tile
