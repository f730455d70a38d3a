"""kv_append_rope's block-wise kernel (taken for batches of long chunks: at
most 64 sequences, at least 512 tokens and 32 per sequence) against the
per-token kernel (the same tokens appended in calls of fewer than 512), bit
for bit: the rotated queries and both arenas.  The batch has chunks that start
and end inside a block, a RoPE table that ends inside a block (positions past
it are skipped) and an invalid block-table entry (its tokens' queries are
rotated, nothing is written)."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import paged_kv_chunked_amd as pkv  # noqa: E402

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built")
    pkv.lib()


def bits(t):
    return t.cpu().numpy().view(np.uint16)


def run(seqs, rope_rows, seed, bad=None):
    """seqs: (P, C) per sequence; bad: (sequence, block index) whose table
    entry is -1.  Returns (one call, per-sequence calls of < 512 tokens), each
    (rotated queries, K arena, V arena)."""
    dev = "cuda"
    rng = np.random.default_rng(seed)
    need = [(P + C + 15) // 16 for P, C in seqs]
    num_blocks = sum(need) + 7
    maxb = max(need)
    ids = rng.permutation(num_blocks)
    bt = np.full((len(seqs), maxb), -1, np.int32)
    o = 0
    for b, n in enumerate(need):
        bt[b, :n] = ids[o:o + n]
        o += n
    if bad is not None:
        bt[bad] = -1
    T = sum(C for _, C in seqs)
    q = torch.from_numpy(rng.standard_normal((T, HQ, D)).astype(np.float16)).to(dev)
    k = torch.from_numpy(rng.standard_normal((T, HKV, D)).astype(np.float16)).to(dev)
    v = torch.from_numpy(rng.standard_normal((T, HKV, D)).astype(np.float16)).to(dev)
    arena0 = rng.integers(0, 65536, (num_blocks, HKV, 16 * D), dtype=np.uint16)
    fill = torch.from_numpy(rng.integers(0, 65536, (T, HQ, D), dtype=np.uint16)).to(dev)
    g = pkv.geom(num_blocks, HKV, HQ, D)
    rope = torch.empty(pkv.pkv_rope_table_bytes(D, rope_rows), dtype=torch.uint8, device=dev)
    pkv.pkv_rope_table_init(rope, 5.0e5, D, rope_rows)
    cu = np.concatenate([[0], np.cumsum([C for _, C in seqs])]).astype(np.int32)

    def fresh():
        ka = torch.from_numpy(arena0.copy()).to(dev).view(torch.float16)
        va = torch.from_numpy(arena0[::-1].copy()).to(dev).view(torch.float16)
        return ka, va, fill.clone().view(torch.float16)

    # one call
    ka, va, qo = fresh()
    pkv.kv_append_rope(g, q, k, v, ka, va, torch.from_numpy(bt).to(dev),
                       torch.from_numpy(cu).to(dev),
                       torch.tensor([P for P, _ in seqs], dtype=torch.int32, device=dev),
                       rope, rope_rows, q_out=qo)
    one = (qo, ka, va)
    # per sequence, in calls of at most 300 tokens
    ka, va, qo = fresh()
    for b, (P, C) in enumerate(seqs):
        for off in range(0, C, 300):
            n = min(300, C - off)
            t0 = int(cu[b]) + off
            pkv.kv_append_rope(g, q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n], ka, va,
                               torch.from_numpy(bt[b:b + 1].copy()).to(dev),
                               torch.tensor([0, n], dtype=torch.int32, device=dev),
                               torch.tensor([P + off], dtype=torch.int32, device=dev),
                               rope, rope_rows, q_out=qo[t0:t0 + n])
    torch.cuda.synchronize()
    return one, (qo, ka, va), fill.cpu().numpy()


@pytest.mark.parametrize("case", [
    # chunks starting and ending inside blocks; the last one past the table's
    # end (650 rows: position 650 is slot 10 of block 40)
    dict(seqs=[(5, 300), (16, 256), (100, 37), (0, 700)], rope_rows=650, seed=1),
    # one invalid block-table entry (sequence 1, block 20)
    dict(seqs=[(0, 512), (48, 480), (3, 61)], rope_rows=2048, seed=2, bad=(1, 20)),
])
def test_block_append_matches_per_token(case):
    one, per, fill = run(**case)
    for name, a, b in zip(("rotated queries", "K arena", "V arena"), one, per):
        assert np.array_equal(bits(a), bits(b)), name
    # every token's query is written, but for positions past the table's end
    qo = bits(one[0])
    t0 = 0
    for P, C in case["seqs"]:
        for t in range(C):
            kept = np.array_equal(qo[t0 + t], fill[t0 + t])
            assert kept == (P + t >= case["rope_rows"]), (P, t)
        t0 += C
