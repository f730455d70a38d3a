"""Host logic of the rocprofv3 summaries (no GPU): how launch durations of one
(kernel, grid) are grouped, and that a traffic record is used only while the
kernel sources it was taken from are unchanged."""
import json

from paged_kv_chunked_amd import rocprof_summary as rs


def test_split_clusters_keeps_one_workload_together():
    durs = [150.0, 139.5, 181.3, 160.2]  # one workload: spread under 1.5x
    assert rs.split_clusters(durs) == [sorted(durs)]


def test_split_clusters_separates_workloads_sharing_a_grid():
    short, long_ = [139.5, 150.4, 181.3], [1632.4, 1682.3, 1850.1]
    groups = rs.split_clusters(long_ + short)
    assert groups == [sorted(short), sorted(long_)]
    # three clusters, cut at each gap of more than 1.5x
    assert rs.split_clusters([1, 1.2, 10, 11, 100]) == [[1, 1.2], [10, 11], [100]]
    assert rs.split_clusters([56.0, 80.0, 137.0, 178.0]) == [[56.0, 80.0], [137.0, 178.0]]


def test_traffic_record_needs_matching_sources(tmp_path):
    call = "paged_attention_decode"
    files = rs.CALLS[call][1]
    rec = {"calls": {call: {"fetch_bytes_per_call": 600.0, "write_bytes_per_call": 8.0,
                            "sources_sha256": rs.sources_sha(files), "sources": list(files)}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    assert rs.load_traffic(str(path), call) == 608.0
    rec["calls"][call]["sources_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert rs.load_traffic(str(path), call) is None


def _fake_db(path, dispatches):
    """A database with the two rocprofv3 views the summaries read."""
    import sqlite3
    c = sqlite3.connect(path)
    c.execute("create table kernels (dispatch_id, name, grid_x, grid_y, grid_z, duration)")
    c.execute("create table pmc_events (dispatch_id, name, counter_name, counter_value)")
    for did, name, grid, dur, cnt in dispatches:
        c.execute("insert into kernels values (?, ?, ?, 1, 1, ?)", (did, name, grid, dur))
        for k, v in cnt.items():  # two instances per counter
            if k.startswith("GRBM_"):  # each instance counts the same active cycles
                rows = (v, 0.9 * v)
            else:                      # per-instance shares of the total
                rows = (v / 2, v / 2)
            for x in rows:
                c.execute("insert into pmc_events values (?, ?, ?, ?)", (did, name, k, x))
    c.commit()


def test_counters_derive_mfma_busy_and_flops(tmp_path):
    cnt = {"SQ_VALU_MFMA_BUSY_CYCLES": 512.0 * 1000, "GRBM_GUI_ACTIVE": 1000.0,
           "SQ_INSTS_VALU_MFMA_MOPS_F16": 2.0e6}
    long_cnt = dict(cnt, GRBM_GUI_ACTIVE=4000.0)
    db = str(tmp_path / "run.db")
    _fake_db(db, [(1, "chunk_mfma_kernel", 512, 140_000.0, cnt),
                  (2, "chunk_mfma_kernel", 512, 150_000.0, cnt),
                  (3, "chunk_mfma_kernel", 512, 1_700_000.0, long_cnt),  # same grid, 10x longer
                  (4, "other_kernel", 64, 5_000.0, cnt)])
    rec = rs.counters(db, str(tmp_path / "out.json"), "cmd", ["chunk_mfma"], simds=1024,
                      flops={"512x1x1 #1": 1.0e9})
    ks = rec["kernels"]
    assert [k["grid"] for k in ks] == ["512x1x1 #1", "512x1x1 #2"]
    short = ks[0]
    assert short["dispatches"] == 2 and short["avg_duration_us"] == 145.0
    assert short["mfma_busy_pct"] == 50.0          # 512e3 / (1000 * 1024)
    assert short["mfma_f16_flop"] == 2.0e6 * 512
    assert short["mfma_f16_flop_over_algorithmic"] == 2.0e6 * 512 / 1.0e9
    assert ks[1]["mfma_busy_pct"] == 12.5 and "mfma_f16_flop_over_algorithmic" not in ks[1]


def test_stats_rows_fold_rare_grids():
    """Timed kernels keep one row per grid; set-up launches whose grids recur
    fewer than five times fold into one row per kernel."""
    rows = [("decode", 5632, 64, 1, 100_000 + i) for i in range(20)]
    rows += [("append", 256 * n, 1, 1, 3_000) for n in range(1, 40)]    # fills: one launch each
    rows += [("append", 1024, 4, 1, 30_000) for _ in range(10)]          # the timed append
    agg = rs.stats_rows(rows)
    assert sorted(agg) == [("append", "1024x4x1"), ("append", "other grids (39)"),
                           ("decode", "5632x64x1")]
    assert len(agg[("append", "other grids (39)")]) == 39
    assert len(agg[("decode", "5632x64x1")]) == 20
