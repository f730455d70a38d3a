"""paged_attention_decode_append (the decode step's append and attention in one
call) against kv_append_rope followed by paged_attention_decode, on the same
seeded workloads over fp16, INT8 and INT4 arenas: outputs, rotated queries and
K/V arena bytes bit for bit; and the fused call's outputs against the oracle on
the edge-length batch."""
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
    print(f"[gpu-append] {msg}", flush=True)


def bits(t):
    a = t.cpu().numpy()
    if a.dtype == np.uint8:
        return a
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


def quant(w, kv_bits):
    """The same workload over INT8 / INT4 arenas (kv_bits 0: fp16)."""
    return dataclasses.replace(w, name=f"{w.name}_i{kv_bits}", kv_bits=kv_bits) if kv_bits else w


def edge_lengths():
    """Contexts 1 (the new token alone), block and pair edges (15 .. 33), split
    edges (383 .. 385, 768, 769) and longer ones; Hq 32 / Hkv 8, fp16."""
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 100, 383, 384, 385, 768, 769, 1000, 2049]
    return workloads.build("append_edges", 21, "f16", 32, 8, 128, 5.0e5,
                           [(L - 1, 1) for L in lens], max_blocks_per_seq=130)


def compare(w, rope_rows=None):
    """rope_rows: pass only that many rows of the rotation table to both calls
    (positions at or past it skip the append)."""
    say(f"{w.name}: separate calls")
    a = harness.DeviceWorkload(w)
    if rope_rows:
        a.rope_max_pos = rope_rows
    a.step()
    say(f"{w.name}: fused call")
    b = harness.DeviceWorkload(w)
    if rope_rows:
        b.rope_max_pos = rope_rows
    b.decode_append()
    torch.cuda.synchronize()
    assert np.array_equal(bits(a.dec_q), bits(b.dec_q)), "rotated queries differ"
    assert np.array_equal(bits(a.k_arena), bits(b.k_arena)), "K arena differs"
    assert np.array_equal(bits(a.v_arena), bits(b.v_arena)), "V arena differs"
    assert np.array_equal(bits(a.dec_out), bits(b.dec_out)), "outputs differ"
    say(f"{w.name}: {b.dec_out.numel()} outputs, queries and arenas bit for bit")
    return b


@pytest.mark.parametrize("kv_bits", [0, 8, 4])
def test_fused_matches_separate_decode_batch(kv_bits):
    compare(quant(workloads.decode_batch(), kv_bits))


def test_fused_matches_separate_shard():
    """One GPU's share of a KV-head split over 8 GPUs (Hq 4 / Hkv 1)."""
    compare(workloads.tp8_decode_batch())


@pytest.mark.parametrize("kv_bits", [0, 8, 4])
def test_fused_edges_against_oracle(kv_bits):
    w = quant(edge_lengths(), kv_bits)
    b = compare(w)
    st = oscript.run_script(w, materialize=True)
    q_rot = oscript.append_step(w, st)
    assert np.array_equal(bits(b.q), q_rot.view(np.uint16)), "rotated q differs from the oracle"
    cu = b.cu_host
    worst = 0.0
    for r in b.dec_rows:
        exp = oscript.attend_row(w, st, r, q_rot[cu[r]:cu[r + 1]], b.scale)[0]
        got = b.dec_out[r - b.dec_rows[0]].cpu().numpy()
        worst = max(worst, float(np.abs(got - exp).max()))
    say(f"{w.name}: max abs error against the oracle {worst:.3e}")
    assert worst <= 2e-3


@pytest.mark.parametrize("hkv,n", [(2, 7), (4, 40)])
def test_fused_matches_separate_few_heads(hkv, n):
    """2 or 4 KV heads (4 query heads each): 2- and 4-wave workgroups, a
    small and a wider batch."""
    lens = [int(x) for x in np.random.default_rng(hkv).integers(1, 4097, n)]
    compare(workloads.build(f"append_hkv{hkv}", 29, "f16", 4 * hkv, hkv, 128, 5.0e5,
                            [(L - 1, 1) for L in lens]))


@pytest.mark.parametrize("kv_bits", [0, 8, 4])
def test_fused_matches_separate_single_splits(kv_bits):
    """Every context within one split: no combine pass, the split kernel
    writes the arena."""
    lens = [1, 7, 16, 33, 200, 383, 384]
    compare(quant(workloads.build("append_short", 23, "f16", 32, 8, 128, 5.0e5,
                                  [(L - 1, 1) for L in lens], max_blocks_per_seq=24), kv_bits))


@pytest.mark.parametrize("kv_bits", [0, 8, 4])
def test_fused_matches_separate_past_table(kv_bits):
    """Positions at or past the table's end (rows of 1000 and more, with 1000
    table rows passed) skip the append in both forms; the rest append."""
    compare(quant(edge_lengths(), kv_bits), rope_rows=1000)


def test_fused_repeated_steps_match():
    """Two fused calls in a row leave the same arena as one (the second writes
    the same bytes), and outputs do not change."""
    w = workloads.decode_batch(num_seqs=9, seed=77)
    b = harness.DeviceWorkload(w)
    b.decode_append()
    torch.cuda.synchronize()
    out1, k1 = bits(b.dec_out), bits(b.k_arena)
    b.decode_append()
    torch.cuda.synchronize()
    assert np.array_equal(out1, bits(b.dec_out)) and np.array_equal(k1, bits(b.k_arena))
