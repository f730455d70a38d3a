"""GPU: paged_attention_mixed, one attention launch for a continuous-batching
step of prefill chunks and decodes (Kshipra part 3, section 5).

Its decode rows (sequences with one new row) must be bit for bit those of
paged_attention_decode and its chunk rows those of paged_attention_chunk
whenever that call does not split keys (paged_attention_chunk_parts = 1; a
split call rounds differently and is checked against the oracle instead);
rows are also checked against the oracle here, and batches whose kinds
interleave (which the separate calls cannot take as one batch) against the
oracle alone.
"""
import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import paged_kv_chunked_amd as pkv  # noqa: E402
from oracle import script as oscript  # noqa: E402
from paged_kv_chunked_amd import harness, workloads  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built")
    pkv.lib()


def say(msg):
    print(f"[gpu-mixed] {msg}", flush=True)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def oracle_rows(w, dw, rows, st=None, q_rot=None, got=None, base=0):
    """max / mean |mixed - oracle| over step rows ``rows`` (every query row);
    ``got`` (packed rows from packed row ``base`` on) instead of the mixed
    output if given."""
    if st is None:
        st = oscript.run_script(w, materialize=False)
        q_rot = oscript.append_step(w, st)
    cu = dw.cu_host
    if got is None:
        got = dw.mix_out.cpu().numpy()
    worst, tot, n = 0.0, 0.0, 0
    for r in rows:
        exp = oscript.attend_row(w, st, r, q_rot[cu[r]:cu[r + 1]], dw.scale)
        d = np.abs(got[cu[r] - base:cu[r + 1] - base].astype(np.float64) - exp)
        worst, tot, n = max(worst, float(d.max())), tot + float(d.sum()), n + d.size
    return worst, tot / max(n, 1)


def check_against_split_calls(w, sample_rows=None):
    say(f"{w.name}: set-up (blocks={w.num_blocks}, step rows={len(w.step)})")
    dw = harness.DeviceWorkload(w)
    dw.step()
    dw.mixed()
    torch.cuda.synchronize()
    mix = dw.mix_out.cpu().numpy()
    cu = dw.cu_host
    say(f"{w.name}: {len(dw.dec_rows)} decode rows, {len(dw.chunk_rows)} chunks")
    if dw.dec_rows:
        dec = dw.dec_out.cpu().numpy()
        for i, r in enumerate(dw.dec_rows):
            assert np.array_equal(bits(mix[cu[r]]), bits(dec[i])), ("decode row", r)
    if dw.chunk_rows:
        chk = dw.chunk_out.cpu().numpy()
        t0, t1 = cu[dw.chunk_rows[0]], cu[dw.chunk_rows[-1] + 1]
        parts = pkv.paged_attention_chunk_parts(dw.g, len(dw.chunk_rows), int(t1 - t0),
                                                dw.chunk_max_ctx)
        if parts == 1:
            assert np.array_equal(bits(mix[t0:t1]), bits(chk)), "chunk rows"
        else:
            rows = dw.chunk_rows if sample_rows is None else \
                [r for r in sample_rows if r in set(dw.chunk_rows)]
            worst, mean = oracle_rows(w, dw, rows, got=chk, base=int(t0))
            say(f"{w.name}: chunk call split into {parts} key parts: oracle max {worst:.2e} "
                f"mean {mean:.2e}")
            assert worst <= 2e-3 and mean <= 2e-4
    rows = range(len(w.step)) if sample_rows is None else sample_rows
    worst, mean = oracle_rows(w, dw, rows)
    say(f"{w.name}: oracle max {worst:.2e} mean {mean:.2e}")
    assert worst <= 2e-3 and mean <= 2e-4
    # a second call (the schedule and its queue counter are rebuilt) gives the
    # same bits
    dw.mix_out.fill_(float("nan"))
    dw.mixed()
    torch.cuda.synchronize()
    assert np.array_equal(bits(dw.mix_out.cpu().numpy()), bits(mix))
    return dw


def test_small_mixed():
    check_against_split_calls(workloads.mixed_step(num_chunks=2, chunk=96, num_decodes=40,
                                                   lo=1, hi=1200, num_sharers=5,
                                                   shared_prefix=256, parent_tokens=264))


def test_decodes_only():
    lens = [1, 2, 15, 16, 17, 383, 384, 385, 768, 769, 1000, 1600, 2049]
    check_against_split_calls(workloads.build("mixed_decodes_only", 21, "f16", 32, 8, 128,
                                              5.0e5, [(L - 1, 1) for L in lens],
                                              max_blocks_per_seq=130))


def test_chunks_only_and_one_row_sequence():
    seqs = [(0, 1), (0, 33), (48, 16), (5, 70), (100, 129), (0, 200), (300, 64), (17, 5)]
    check_against_split_calls(workloads.build("mixed_chunks", 22, "f16", 32, 8, 128, 5.0e5,
                                              seqs, max_blocks_per_seq=40))


def test_short_contexts_need_no_merge():
    """Every context fits one 384-token split: no partials, no combine."""
    seqs = [(10, 1), (383, 1), (200, 1), (0, 40), (64, 100)]
    check_against_split_calls(workloads.build("mixed_one_split", 23, "f16", 32, 8, 128, 5.0e5,
                                              seqs, max_blocks_per_seq=30))


def test_sixteen_kv_heads():
    """Hkv 16: decode units cover the KV heads in two groups of 8 waves."""
    seqs = [(700, 1), (1500, 1), (30, 1), (0, 70), (400, 33)]
    check_against_split_calls(workloads.build("mixed_hkv16", 24, "f16", 64, 16, 128, 5.0e5,
                                              seqs, max_blocks_per_seq=100))


def test_interleaved_kinds_against_oracle():
    seqs = [(300, 1), (0, 70), (1000, 1), (48, 16), (2000, 1), (5, 2), (0, 1), (800, 130)]
    w = workloads.build("mixed_interleaved", 25, "f16", 32, 8, 128, 5.0e5, seqs,
                        max_blocks_per_seq=130)
    say(f"{w.name}: set-up")
    dw = harness.DeviceWorkload(w)
    assert not dw.split_ok
    dw.append()
    dw.mixed()
    torch.cuda.synchronize()
    worst, mean = oracle_rows(w, dw, range(len(seqs)))
    say(f"{w.name}: oracle max {worst:.2e} mean {mean:.2e}")
    assert worst <= 2e-3 and mean <= 2e-4


def test_mixed_full():
    """The 2048-token-budget step: 4 chunks of 256 + 1024 decodes (16 sharing a
    prefix); every row bit for bit against the separate calls, sampled rows
    against the oracle."""
    w = workloads.mixed_step()
    rng = np.random.default_rng(3)
    sample = sorted(set(w.chunk_rows()[:1] +
                        rng.choice(w.decode_rows(), size=8, replace=False).tolist()))
    check_against_split_calls(w, sample_rows=sample)


@pytest.mark.parametrize("kv_bits", [0, 8, 4])
def test_empty_sequences_change_nothing(kv_bits):
    """Sequences with no new rows (a repeated cu_q_lens entry) anywhere in the
    batch leave every output bit of paged_attention_chunk and
    paged_attention_mixed unchanged (fp16, INT8 and INT4 arenas)."""
    seqs = [(300, 1), (0, 70), (1000, 1), (48, 16)]
    w = workloads.build("mixed_empty", 26, "f16", 32, 8, 128, 5.0e5, seqs,
                        max_blocks_per_seq=70)
    if kv_bits:
        w = _quant(w, kv_bits)
    say(f"{w.name}: set-up")
    dw = harness.DeviceWorkload(w)
    dw.append()
    dw.mixed()
    torch.cuda.synchronize()
    ref = dw.mix_out.clone()
    # insert empty sequences before, between and after the real ones
    cu = dw.cu_host.tolist()
    starts = dw.starts_host.tolist()
    bt = dw.bt_host
    order = [None, 0, None, 1, 2, None, 3, None]
    cu2, st2, rows = [0], [], []
    for o in order:
        if o is None:
            cu2.append(cu2[-1])
            st2.append(0)
            rows.append(np.full(bt.shape[1], -1, np.int32))
        else:
            cu2.append(cu2[-1] + cu[o + 1] - cu[o])
            st2.append(starts[o])
            rows.append(bt[o])
    dev = dw.device
    cu2 = torch.tensor(cu2, dtype=torch.int32, device=dev)
    st2 = torch.tensor(st2, dtype=torch.int32, device=dev)
    bt2 = torch.from_numpy(np.stack(rows)).to(dev)
    out = torch.full_like(ref, float("nan"))
    pkv.paged_attention_mixed(dw.g, out, dw.q, dw.k_arena, dw.v_arena, bt2, cu2, st2,
                              dw.mix_max_q, dw.mix_max_ctx, dw.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out.cpu().numpy()), bits(ref.cpu().numpy()))
    # the chunk call over the same batch: compare with its own run without the
    # empty sequences
    cu1 = torch.tensor(cu, dtype=torch.int32, device=dev)
    ref_c = torch.full_like(ref, float("nan"))
    pkv.paged_attention_chunk(dw.g, ref_c, dw.q, dw.k_arena, dw.v_arena, dw.bt, cu1, dw.starts,
                              dw.mix_max_q, dw.mix_max_ctx, dw.scale)
    out_c = torch.full_like(ref, float("nan"))
    pkv.paged_attention_chunk(dw.g, out_c, dw.q, dw.k_arena, dw.v_arena, bt2, cu2, st2,
                              dw.mix_max_q, dw.mix_max_ctx, dw.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_c.cpu().numpy()), bits(ref_c.cpu().numpy()))


def _quant(w, bits):
    return dataclasses.replace(w, name=f"{w.name}_i{bits}", kv_bits=bits)


@pytest.mark.parametrize("bits", [8, 4])
def test_small_mixed_quant(bits):
    """INT8 / INT4 arenas: the mixed kernel's quantized chunk and decode units
    against the quantized stand-alone calls, bit for bit."""
    check_against_split_calls(_quant(workloads.mixed_step(num_chunks=2, chunk=96,
                                                          num_decodes=40, lo=1, hi=1200,
                                                          num_sharers=5, shared_prefix=256,
                                                          parent_tokens=264), bits))


@pytest.mark.parametrize("bits", [8, 4])
def test_mixed_full_quant(bits):
    w = _quant(workloads.mixed_step(), bits)
    rng = np.random.default_rng(4)
    sample = sorted(set(w.chunk_rows()[:1] +
                        rng.choice(w.decode_rows(), size=6, replace=False).tolist()))
    check_against_split_calls(w, sample_rows=sample)
