"""GPU: decode over shared prefixes (Kshipra part 3, section 3).

paged_attention_decode_shared reads the leading splits that groups of rows
share once per 4 rows; its output must be bit for bit paged_attention_decode's
(which the parity tests check against the oracle), and is also checked against
the oracle here on sampled rows.
"""
import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import paged_kv_chunked_amd as pkv  # noqa: E402
from oracle import script as oscript  # noqa: E402
from paged_kv_chunked_amd import harness, workloads  # noqa: E402
from paged_kv_chunked_amd.workloads import StepSeq, Workload, _blocks, _round_robin  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpkv.so is not built")
    pkv.lib()


def say(msg):
    print(f"[gpu-shared] {msg}", flush=True)


def two_prompts(seed=77, heads=(32, 8)):
    """Rows 0-4 continue an 800-token prompt, rows 5-6 a 416-token one, rows 7-8
    are independent: groups of 5, 2, 1, 1 (skips 2, 1, 0, 0).  ``heads`` =
    (query heads, KV heads)."""
    rng = np.random.default_rng(seed)
    prompts = [(800, 5), (416, 2)]
    seqs, parents, pool_seqs = [], [], 0
    for plen, n in prompts:
        for _ in range(n):
            seqs.append((plen + int(rng.integers(1, 300)) - 1, plen))
    for _ in range(2):
        seqs.append((int(rng.integers(100, 1500)) - 1, 0))
    S = len(seqs)
    parent_ids = [S, S + 1]
    need = [_blocks(p + 1) - (pl // 16) for p, pl in seqs]
    num_blocks = int(math.ceil(1.1 * (sum(need) + sum(pl // 16 for pl, _ in prompts))))
    script = [("shuffle", rng.permutation(num_blocks).astype(np.int64))]
    fi = 0
    for (plen, _), pid in zip(prompts, parent_ids):
        script += [("alloc", np.full(plen // 16, pid, np.int64)), ("fill", fi, pid, 0, plen)]
        fi += 1
    row = 0
    for (plen, n), pid in zip(prompts, parent_ids):
        for _ in range(n):
            script.append(("fork", row, pid))
            row += 1
        script.append(("release", pid))
    script.append(("alloc", _round_robin(need, range(S))))
    for b, (p, pl) in enumerate(seqs):
        if p > pl:
            script.append(("fill", fi, b, pl, p - pl))
            fi += 1
    step = tuple(StepSeq(b, p, 1) for b, (p, _) in enumerate(seqs))
    return Workload(name=f"two_prompts_{heads[0]}q{heads[1]}kv", seed=seed, dtype="f16",
                    num_q_heads=heads[0], num_kv_heads=heads[1],
                    head_dim=128, theta=5.0e5, num_blocks=num_blocks, max_blocks_per_seq=120,
                    num_pool_seqs=S + 2, script=script, step=step)


def partials(dw):
    """The decode workspace as (o [S, nsplit, Hq, D], m_l [S, nsplit, Hq, 2])."""
    S, Hq, D = len(dw.dec_rows), dw.w.num_q_heads, dw.w.head_dim
    nsplit = -(-dw.dec_max_len // pkv.DECODE_SPLIT)
    parts = S * nsplit * Hq
    ws = dw.dec_ws.cpu().numpy().view(np.float32)
    off = ((parts * D * 4 + 255) & ~255) // 4
    return (ws[:parts * D].reshape(S, nsplit, Hq, D).copy(),
            ws[off:off + 2 * parts].reshape(S, nsplit, Hq, 2).copy())


def check(w, sample_rows):
    say(f"{w.name}: set-up")
    dw = harness.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    plain = dw.dec_out.cpu().numpy().copy()
    po, pml = partials(dw)
    dw.dec_out.fill_(float("nan"))
    dw.decode_shared()
    torch.cuda.synchronize()
    shared = dw.dec_out.cpu().numpy()
    so, sml = partials(dw)
    say(f"{w.name}: groups {np.diff(dw.dec_group_start.cpu().numpy()).tolist()}, "
        f"skips {sorted(set(dw.dec_row_skip.cpu().numpy().tolist()))}")
    assert dw.dec_max_skip > 0
    skip = dw.dec_row_skip.cpu().numpy()
    bad_o = np.argwhere((po.view(np.uint32) != so.view(np.uint32)).any(axis=3))
    bad_ml = np.argwhere((pml.view(np.uint32) != sml.view(np.uint32)).any(axis=3))
    bad_out = np.argwhere((plain.view(np.uint32) != shared.view(np.uint32)).any(axis=2))
    if len(bad_out) or len(bad_o) or len(bad_ml):
        say(f"differing outputs (row, head): {len(bad_out)}, first {bad_out[:8].tolist()}; "
            f"nan in shared {int(np.isnan(shared).sum())}")
        for name, bad, a, b in (("o", bad_o, po, so), ("m_l", bad_ml, pml, sml)):
            rows_splits = sorted({(int(r), int(s)) for r, s, _ in bad})
            say(f"differing partials {name}: {len(bad)} (row, split, head); (row, split) "
                f"{rows_splits[:12]}; skips of those rows "
                f"{sorted({int(skip[r]) for r, _ in rows_splits})}")
            for r, sp, h in bad[:4]:
                say(f"  {name}[{r},{sp},{h}] plain {a[r, sp, h, :4].tolist()} "
                    f"shared {b[r, sp, h, :4].tolist()}")
    assert np.array_equal(plain.view(np.uint32), shared.view(np.uint32))
    st = oscript.run_script(w, materialize=False)
    q_rot = oscript.append_step(w, st)
    for r in sample_rows:
        exp = oscript.attend_row(w, st, r, q_rot[r:r + 1], dw.scale)[0]
        d = np.abs(shared[r].astype(np.float64) - exp)
        assert d.max() <= 2e-3 and d.mean() <= 2e-4, (r, d.max(), d.mean())
    return dw


def test_two_prompts_bitwise_equal_to_decode():
    check(two_prompts(), sample_rows=[0, 4, 5, 8])


# Workgroups of 4, 2 and 1 KV heads (the shared units then hold 1 head x 4, 2
# and 1 quads), 16 KV heads (two head groups), and 3 KV heads, whose
# workgroup width the shared units do not take (the call computes every split
# per row, the same result).
@pytest.mark.parametrize("heads", [(16, 4), (8, 2), (4, 1), (64, 16), (12, 3)])
def test_two_prompts_other_head_counts(heads):
    check(two_prompts(heads=heads), sample_rows=[0, 5, 8])


def test_one_shared_system_prompt():
    dw = check(workloads.shared_prefix_decode(), sample_rows=[0, 31, 63])
    assert np.diff(dw.dec_group_start.cpu().numpy()).tolist() == [64]
