"""GPU: preemption by swapping (Kshipra part 3, section 5).

A decode batch runs (fp16, INT8 and INT4 arenas); one sequence's blocks are
swapped out to pinned host memory (pkv_swap_out), compared bit for bit with
the oracle's packed tiles,
its old blocks are overwritten, and the tiles are swapped back in
(pkv_swap_in) into freshly allocated blocks.  With the block-table row
pointing at the new blocks, the decode output must be bit for bit the output
before preemption (the kernels never depend on physical block ids).
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
    print(f"[gpu-swap] {msg}", flush=True)


@pytest.mark.parametrize("kv_bits", [0, 8, 4])
def test_swap_out_in_roundtrip_bitwise(kv_bits):
    w = dataclasses.replace(workloads.decode_batch(num_seqs=8, lo=100, hi=900, seed=2024),
                            kv_bits=kv_bits)
    say(f"set-up (kv_bits={kv_bits})")
    dw = harness.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    out0 = dw.dec_out.cpu().numpy().copy()

    r = int(np.argmin(dw.dec_lens_host))   # shortest: fits in the arena's spare blocks
    L = int(dw.dec_lens_host[r])
    nblk = -(-L // 16)
    old = dw.bt_host[r, :nblk].astype(np.int32).copy()
    g = dw.g
    nbytes = pkv.pkv_swap_bytes(g, nblk)
    buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    ids = torch.from_numpy(old).to(dw.device)
    say(f"swap out {nblk} blocks ({nbytes} bytes) to pinned host memory")
    pkv.pkv_swap_out(g, dw.k_arena, dw.v_arena, ids, buf)
    torch.cuda.synchronize()

    st = oscript.run_script(w)
    oscript.append_step(w, st)
    exp = st.arena.swap_out(old)
    assert np.array_equal(buf.numpy(), exp)

    # the sequence is preempted: it is restored into other blocks, and its
    # old blocks are overwritten (all-ones bytes: NaN in fp16, NaN scales in
    # quantized arenas) and freed
    assert dw.pool.num_free >= nblk
    new = np.array([dw.pool.alloc() for _ in range(nblk)], dtype=np.int32)[::-1].copy()
    assert not set(new.tolist()) & set(old.tolist())
    junk = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dw.device)
    pkv.pkv_swap_in(g, dw.k_arena, dw.v_arena, ids, junk)
    for b in old:
        dw.pool.decref(int(b))
    say("swap in to fresh blocks")
    pkv.pkv_swap_in(g, dw.k_arena, dw.v_arena, torch.from_numpy(new).to(dw.device), buf)
    # re-read: the restored tiles equal the oracle's
    back = torch.empty(nbytes, dtype=torch.uint8, device=dw.device)
    pkv.pkv_swap_out(g, dw.k_arena, dw.v_arena, torch.from_numpy(new).to(dw.device), back)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), exp)

    row = dw.bt_host[r].copy()
    row[:nblk] = new
    dw.dec_bt[r] = torch.from_numpy(row).to(dw.device)
    dw.decode()
    torch.cuda.synchronize()
    out1 = dw.dec_out.cpu().numpy()
    assert np.array_equal(out0.view(np.uint32), out1.view(np.uint32))
