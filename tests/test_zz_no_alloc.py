"""GPU: paged_attention_decode_noalloc, the allocation-free variant of
paged_attention_decode (split partials in the library's static per-GPU scratch
array), called through the C ABI, against paged_attention_decode on the same
inputs: bit for bit, on two calls in a row (the second smaller, so the scratch
still holds the first call's partials) and over an INT8 arena."""
import ctypes
import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import paged_kv_chunked_amd as pkv  # noqa: E402
from paged_kv_chunked_amd import harness, workloads  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built")
    pkv.lib()


def noalloc_call(dw, out):
    """paged_attention_decode_noalloc through the C ABI (ctypes, no binding)."""
    lib = pkv.lib()
    rc = lib.paged_attention_decode_noalloc(
        ctypes.byref(dw.g), out.data_ptr(), pkv.F32, dw.dec_q.data_ptr(), dw.k_arena.data_ptr(),
        dw.v_arena.data_ptr(), dw.dec_bt.data_ptr(), dw.dec_bt.shape[1], dw.dec_lens.data_ptr(),
        dw.dec_lens.shape[0], dw.dec_max_len, ctypes.c_float(dw.scale),
        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, pkv.STATUS.get(rc, rc)


def check(w):
    print(f"[no-alloc] {w.name}: {len(w.step)} decode rows", flush=True)
    dw = harness.DeviceWorkload(w)
    dw.step()                        # append + paged_attention_decode (workspace)
    torch.cuda.synchronize()
    ref = dw.dec_out.cpu().numpy()
    assert np.isfinite(ref).all()
    out = torch.full_like(dw.dec_out, float("nan"))
    noalloc_call(dw, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), w.name
    return dw


def test_noalloc_matches_decode_two_calls():
    big = workloads.decode_batch()                                    # 64 x U[512, 4096]
    small = workloads.decode_batch(num_seqs=9, lo=1, hi=1500, seed=77)
    dw = check(big)
    need = pkv.paged_attention_decode_workspace_bytes(dw.g, len(big.step), dw.dec_max_len)
    assert 0 < need <= 32 << 20
    del dw
    check(small)                                                      # scratch holds big's partials


def test_noalloc_int8_arena():
    w = dataclasses.replace(workloads.decode_batch(num_seqs=12, lo=300, hi=5000, seed=78),
                            kv_bits=8, name="decode_noalloc_i8")
    check(w)
