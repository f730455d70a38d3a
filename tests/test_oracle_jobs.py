"""The worker-process oracle the large GPU parity cases use gives what the
plain oracle gives: expected outputs equal to attend_row's, and block digests
equal to those of the materialised oracle arena's blocks (CPU only)."""
import dataclasses

import numpy as np
import pytest

import oracle_jobs
from oracle import script as oscript
from paged_kv_chunked_amd import workloads


def small_mixed(bits=0):
    w = workloads.mixed_step(num_chunks=2, chunk=40, num_decodes=12, lo=1, hi=300,
                             num_sharers=3, shared_prefix=64, parent_tokens=72)
    return dataclasses.replace(w, kv_bits=bits, name=f"{w.name}_{bits}")


@pytest.mark.parametrize("bits", [0, 8, 4])
def test_jobs_match_plain_oracle(bits):
    w = small_mixed(bits)
    scale = 1.0 / np.sqrt(w.head_dim)
    sym = oscript.run_script(w, materialize=False)
    q_rot = oscript.append_step(w, sym)
    mat = oscript.run_script(w, materialize=True)
    assert np.array_equal(oscript.append_step(w, mat).view(np.uint16), q_rot.view(np.uint16))
    cu = np.concatenate([[0], np.cumsum([s.count for s in w.step])])
    rows3 = np.array([0, 7, 39])
    jobs = [(r, None, True) for r in w.decode_rows()[:5]] + \
           [(w.chunk_rows()[0], rows3, True), (w.chunk_rows()[1], None, False)]
    out = oracle_jobs.run(w, sym, q_rot, cu, jobs, scale, workers=2)
    assert [o[0] for o in out] == [j[0] for j in jobs]
    for (r, rows, blocks), (r2, rows2, exp, dk, dv) in zip(jobs, out):
        ref = oscript.attend_row(w, mat, r, q_rot[cu[r]:cu[r + 1]], scale, rows=rows)
        assert np.array_equal(exp, ref)
        if not blocks:
            assert dk is None and dv is None
            continue
        s = w.step[r]
        nb = -(-(s.start + s.count) // w.block_size)
        table = mat.tables[s.seq][:nb]
        if bits:
            kimg, vimg = mat.arena.image("k", table), mat.arena.image("v", table)
        else:
            kimg, vimg = mat.arena.k[table], mat.arena.v[table]
        assert oracle_jobs.digest(kimg) == dk
        assert oracle_jobs.digest(vimg) == dv
