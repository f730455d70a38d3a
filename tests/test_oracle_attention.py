"""Pins for oracle.attention and oracle.script (CPU only).

Each check would fail for a plausible slip in the oracle (dropped scale, a
strict mask, the wrong GQA head map, a transposed operand, no max shift, a
chunk rotated from 0 instead of P):
  (i)    the pages' own per-row online-softmax loop over blocks read through a
         block table (Kshipra part 3, section 4), run in fp64;
  (ii)   output unchanged under any permutation of physical block ids;
  (iii)  uniform V returns V;  (iv) a single key returns its V exactly;
  (v)    q = 0 returns the mean of the visible V rows;
  (vi)   a decode at position L-1 equals the last row of a chunk ending at L;
  (vii)  batch invariance holds by construction here (each sequence is its own
         computation); it is checked on the GPU path;
  (viii) torch's scaled_dot_product_attention in fp64 with an explicit mask
         and enable_gqa (a library routine);
  (ix)   GQA equals MHA after repeating each KV head for its query group;
  (x)    brute force with scalar math.exp loops on tiny hypothesis shapes;
  plus chunked = dense: RoPE at absolute positions makes the chunk rows of a
  prefix + chunk run equal the same rows of one dense pass over the sequence,
  and a 512-row chunk equals two 256-row chunks with an append in between.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import arena, attention, pool, rope, script
from paged_kv_chunked_amd import workloads

SCALE = lambda D: float(np.float32(1.0 / math.sqrt(D)))  # noqa: E731


def _qkv(rng, C, L, Hq, Hkv, D, dtype=np.float64):
    q = rng.standard_normal((C, Hq, D)).astype(dtype)
    K = rng.standard_normal((L, Hkv, D)).astype(dtype)
    V = rng.standard_normal((L, Hkv, D)).astype(dtype)
    return q, K, V


def pages_block_loop(q, K, V, start, scale, block=16):
    """Kshipra part 3, section 4: per query row, a running max m, denominator l
    and accumulator o over (k_blk, v_blk) blocks, then out = o / l.  Keys past
    the row's causal frontier are left out of each block."""
    C, Hq, D = q.shape
    G = Hq // K.shape[1]
    out = np.empty((C, Hq, D))
    for i in range(C):
        for h in range(Hq):
            g = h // G
            n = start + i + 1
            m, l, o = -math.inf, 0.0, np.zeros(D)
            for b0 in range(0, n, block):
                kb = K[b0:min(n, b0 + block), g].astype(np.float64)
                vb = V[b0:min(n, b0 + block), g].astype(np.float64)
                s = kb @ q[i, h].astype(np.float64) * scale
                m_new = max(m, s.max())
                p = np.exp(s - m_new)
                l = l * math.exp(m - m_new) + p.sum()
                o = o * math.exp(m - m_new) + p @ vb
                m = m_new
            out[i, h] = o / l
    return out


def brute(q, K, V, start, scale):
    C, Hq, D = q.shape
    G = Hq // K.shape[1]
    out = np.zeros((C, Hq, D))
    for i in range(C):
        for h in range(Hq):
            n = start + i + 1
            s = [sum(float(q[i, h, d]) * float(K[j, h // G, d]) for d in range(D)) * scale
                 for j in range(n)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = sum(w)
            for d in range(D):
                out[i, h, d] = sum(w[j] * float(V[j, h // G, d]) for j in range(n)) / tot
    return out


def test_pages_online_block_loop():
    rng = np.random.default_rng(1)
    for C, P, Hq, Hkv, D in [(16, 48, 4, 2, 64), (5, 0, 8, 2, 16), (33, 70, 4, 4, 32), (1, 200, 4, 1, 8)]:
        q, K, V = _qkv(rng, C, P + C, Hq, Hkv, D)
        ref = pages_block_loop(q, K, V, P, SCALE(D))
        got = attention.attend(q, K, V, P, SCALE(D))
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@settings(max_examples=40, deadline=None)
@given(hkv=st.sampled_from([1, 2]), g=st.sampled_from([1, 2, 4]), D=st.sampled_from([2, 4, 8]),
       C=st.integers(1, 6), P=st.integers(0, 40), seed=st.integers(0, 2 ** 31))
def test_brute_force_tiny(hkv, g, D, C, P, seed):
    rng = np.random.default_rng(seed)
    q, K, V = _qkv(rng, C, P + C, hkv * g, hkv, D)
    np.testing.assert_allclose(attention.attend(q, K, V, P, 0.7), brute(q, K, V, P, 0.7),
                               rtol=0, atol=1e-12)


def test_sdpa_fp64_with_explicit_mask():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(4)
    C, P, Hq, Hkv, D = 40, 100, 8, 2, 64
    q, K, V = _qkv(rng, C, P + C, Hq, Hkv, D)
    got = attention.attend(q, K, V, P, 1.0 / math.sqrt(D))
    L = P + C
    mask = torch.from_numpy(np.arange(L)[None, :] <= (P + np.arange(C))[:, None])
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(K).permute(1, 0, 2)[None],
        torch.from_numpy(V).permute(1, 0, 2)[None], attn_mask=mask, enable_gqa=True)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_gqa_equals_mha_repeat():
    rng = np.random.default_rng(5)
    q, K, V = _qkv(rng, 7, 30, 8, 2, 16)
    got = attention.attend(q, K, V, 23, 0.3)
    mha = attention.attend(q, np.repeat(K, 4, axis=1), np.repeat(V, 4, axis=1), 23, 0.3)
    assert np.array_equal(got, mha)


def test_uniform_v_returns_v():
    rng = np.random.default_rng(6)
    q, K, _ = _qkv(rng, 9, 50, 4, 2, 32)
    u = rng.standard_normal(32)
    V = np.broadcast_to(u, (50, 2, 32)).copy()
    out = attention.attend(q, K, V, 41, 0.2)
    np.testing.assert_allclose(out, np.broadcast_to(u, out.shape), rtol=0, atol=1e-14)


def test_single_key_returns_its_v_exactly():
    rng = np.random.default_rng(7)
    q, K, V = _qkv(rng, 1, 1, 4, 2, 64, np.float16)
    out = attention.attend(q, K, V, 0, SCALE(64))
    for h in range(4):
        assert np.array_equal(out[0, h], V[0, h // 2].astype(np.float64))


def test_zero_query_is_mean_of_visible_rows():
    rng = np.random.default_rng(8)
    _, K, V = _qkv(rng, 6, 40, 4, 2, 16)
    q = np.zeros((6, 4, 16))
    out = attention.attend(q, K, V, 34, 0.5)
    for i in range(6):
        for h in range(4):
            np.testing.assert_allclose(out[i, h], V[:35 + i, h // 2].mean(axis=0), atol=1e-14)


def test_decode_equals_last_chunk_row():
    rng = np.random.default_rng(9)
    q, K, V = _qkv(rng, 16, 64, 4, 2, 64)
    chunk = attention.attend(q, K, V, 48, 0.125)
    dec = attention.attend_decode(q[-1], K, V, 64, 0.125)
    np.testing.assert_allclose(dec, chunk[-1], rtol=0, atol=1e-15)


def test_block_id_permutation_invariance():
    rng = np.random.default_rng(10)
    N, H, D, L = 20, 2, 16, 70
    K = rng.standard_normal((L, H, D)).astype(np.float16)
    V = rng.standard_normal((L, H, D)).astype(np.float16)
    q = rng.standard_normal((1, 4, D)).astype(np.float16)
    outs = []
    for seed in range(3):
        t = np.random.default_rng(100 + seed).permutation(N)[:5]
        a = arena.Arena(N, H, D, np.float16)
        a.write(t, 0, K, V)
        Kg, Vg = a.gather(t, L)
        outs.append(attention.attend(q, Kg, Vg, L - 1, 0.25))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_large_scores_no_overflow():
    rng = np.random.default_rng(12)
    q, K, V = _qkv(rng, 4, 30, 2, 1, 8)
    out = attention.attend(q * 300.0, K, V, 26, 1.0)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, brute(q * 300.0, K, V, 26, 1.0), atol=1e-12)


# ---------------------------------------------------------------------------
# chunked = dense through the whole oracle pipeline (pool, arena, RoPE)
# ---------------------------------------------------------------------------

def _sequence_dense(w, L, q_all, k_all, v_all, scale):
    """One dense pass: every token rotated at its own position 0..L-1."""
    cos, sin = script.rope_tables(w, L)
    pos = np.arange(L)
    q = rope.rotate_store(q_all, pos, cos, sin, w.np_dtype)
    k = rope.rotate_store(k_all, pos, cos, sin, w.np_dtype)
    return attention.attend(q, k, v_all, 0, scale)


def test_chunk_rows_equal_dense_pass_tiny_workload():
    w = workloads.tiny()
    st_ = script.run_script(w)
    q_rot = script.append_step(w, st_)
    scale = SCALE(w.head_dim)
    got = script.attend_row(w, st_, 0, q_rot, scale)
    # the same raw tokens, as one dense sequence of 64 tokens
    k_pre, v_pre = w.draw_fill(0)
    q_new, k_new, v_new = w.draw_step(0)
    L = 64
    q_all = np.concatenate([np.zeros((48, 4, 64), np.float32), q_new])
    dense = _sequence_dense(w, L, q_all, np.concatenate([k_pre, k_new]),
                            np.concatenate([v_pre, v_new]), scale)
    np.testing.assert_allclose(got, dense[48:], rtol=0, atol=1e-12)
    # rotating the chunk from 0 instead of P breaks the equality
    cos, sin = script.rope_tables(w, L)
    wrong_q = rope.rotate_store(q_new, np.arange(16), cos, sin, w.np_dtype)
    wrong = script.attend_row(w, st_, 0, wrong_q, scale)
    assert np.abs(wrong - dense[48:]).max() > 1e-2


def test_chunk_split_invariance():
    """512 rows at P equal 256 rows at P then 256 rows at P+256."""
    rng = np.random.default_rng(13)
    w = workloads.build("split", 77, "f16", 4, 2, 32, 1.0e4, [(40, 512)], max_blocks_per_seq=40)
    cos, sin = script.rope_tables(w, 600)
    st_ = script.run_script(w, cos_sin=(cos, sin))
    q, k, v = w.draw_step(0)
    pos = 40 + np.arange(512)
    q_r = rope.rotate_store(q, pos, cos, sin, np.float16)
    k_r = rope.rotate_store(k, pos, cos, sin, np.float16)
    table = st_.tables[0]
    st_.arena.write(table, 40, k_r, v)
    K, V = st_.arena.gather(table, 552)
    one = attention.attend(q_r, K, V, 40, 0.2)
    a = attention.attend(q_r[:256], K[:296], V[:296], 40, 0.2)
    b = attention.attend(q_r[256:], K, V, 296, 0.2)
    np.testing.assert_allclose(np.concatenate([a, b]), one, rtol=0, atol=1e-13)
    del rng


def test_symbolic_matches_materialized():
    w = workloads.mixed_step(num_chunks=2, chunk=40, num_decodes=12, lo=20, hi=400,
                             num_sharers=3, shared_prefix=64, parent_tokens=72)
    mat = script.run_script(w)
    sym = script.run_script(w, materialize=False)
    assert mat.tables == sym.tables and mat.copies == sym.copies and len(mat.copies) == 3
    script.append_step(w, mat)
    script.append_step(w, sym)
    for r in range(len(w.step)):
        Km, Vm = script.sequence_kv(w, mat, r)
        Ks, Vs = script.sequence_kv(w, sym, r)
        assert np.array_equal(Km.view(np.uint16), Ks.view(np.uint16))
        assert np.array_equal(Vm.view(np.uint16), Vs.view(np.uint16))


def test_mixed_sharers_see_parent_prefix():
    w = workloads.mixed_step(num_chunks=1, chunk=40, num_decodes=6, lo=20, hi=400,
                             num_sharers=2, shared_prefix=64, parent_tokens=72)
    st_ = script.run_script(w)
    k_par, v_par = w.draw_fill(0)
    cos, sin = script.rope_tables(w)
    k_par_r = rope.rotate_store(k_par, np.arange(72), cos, sin, np.float16)
    sharers = [op[1] for op in w.script if op[0] == "fork"]
    for s in sharers:
        K, V = st_.arena.gather(st_.tables[s], 72)
        assert np.array_equal(K.view(np.uint16), k_par_r.view(np.uint16))
        assert np.array_equal(V.view(np.uint16), v_par.view(np.uint16))
    t0, t1 = (st_.tables[s] for s in sharers)
    assert t0[:4] == t1[:4] and t0[4] != t1[4]           # 64 shared tokens, copied 5th block
    assert all(st_.pool.refcount[b] == 2 for b in t0[:4])
