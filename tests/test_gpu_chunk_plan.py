"""GPU: paged_attention_chunk as its two halves (Kshipra part 3, sections 4
and 5: a step's batch is fixed before its layers run, so its schedule is made
once).  One plan, then runs over two arenas (standing in for two layers: the
K and V arenas, and the same two swapped), each bit for bit the whole call on
the same arena; the whole call's own parity against the oracle is checked in
test_gpu_parity.py.  A run over a schedule holding only out-of-range entries
computes nothing and touches no row.
"""
import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import paged_kv_chunked_amd as pkv  # noqa: E402
from paged_kv_chunked_amd import harness, workloads  # noqa: E402
from test_gpu_parity import generic_shape, i4, i8, small_chunk, split_prefix_three  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built")
    pkv.lib()


def say(msg):
    print(f"[gpu-chunk-plan] {msg}", flush=True)


CASES = {
    "small_chunk": small_chunk,
    "split_prefix_three": split_prefix_three,              # 4 key-range parts
    "small_chunk_i8": lambda: i8(small_chunk()),
    "split_prefix_three_i4": lambda: i4(split_prefix_three()),
    "generic_f16_d64": lambda: generic_shape("generic_f16_d64", "f16", 8, 2, 64),  # no schedule
    "chunk_llama3_8b": workloads.chunk_batch,
}


def bits(t):
    return t.cpu().numpy().view(np.uint32).copy()


@pytest.mark.parametrize("name", list(CASES))
def test_plan_then_runs_equal_whole_calls(name):
    w = CASES[name]()
    say(f"{name}: set-up")
    dw = harness.DeviceWorkload(w)
    dw.step()
    k, v = dw.k_arena, dw.v_arena
    dw.chunk(k_arena=k, v_arena=v)
    torch.cuda.synchronize()
    ref_kv = bits(dw.chunk_out)
    dw.chunk(k_arena=v, v_arena=k)
    torch.cuda.synchronize()
    ref_vk = bits(dw.chunk_out)
    # the plan rewrites the whole schedule
    if dw.chunk_ws is not None:
        dw.chunk_ws.fill_(0x7F)
    dw.chunk_plan()
    for arenas, ref in (((k, v), ref_kv), ((v, k), ref_vk), ((k, v), ref_kv)):
        dw.chunk_out.fill_(float("nan"))
        dw.chunk_run(k_arena=arenas[0], v_arena=arenas[1])
        torch.cuda.synchronize()
        assert np.array_equal(bits(dw.chunk_out), ref), name
    say(f"{name}: three runs over one plan, bit for bit")


def test_run_skips_out_of_range_schedule_entries():
    w = small_chunk()
    dw = harness.DeviceWorkload(w)
    dw.step()
    assert pkv.paged_attention_chunk_parts(dw.g, len(w.step), dw.chunk_q.shape[0],
                                           dw.chunk_max_ctx) == 1
    dw.chunk_ws.fill_(0x7F)          # every entry 0x7F7F7F7F: past the item range
    dw.chunk_out.fill_(float("nan"))
    dw.chunk_run()
    torch.cuda.synchronize()
    assert np.isnan(dw.chunk_out.cpu().numpy()).all()
