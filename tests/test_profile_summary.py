"""Host logic of the rocprofv3 summaries (no GPU): how launch durations of one
(kernel, grid) are grouped, and that a traffic record is used only while the
kernel sources it was taken from are unchanged."""
import json

from paged_kv_chunked_amd import rocprof_summary as rs


def test_split_clusters_keeps_one_workload_together():
    durs = [150.0, 139.5, 181.3, 160.2]  # one workload: spread well under 3x
    assert rs.split_clusters(durs) == [sorted(durs)]


def test_split_clusters_separates_workloads_sharing_a_grid():
    short, long_ = [139.5, 150.4, 181.3], [1632.4, 1682.3, 1850.1]
    groups = rs.split_clusters(long_ + short)
    assert groups == [sorted(short), sorted(long_)]
    # three clusters, cut at each gap of more than 3x
    assert rs.split_clusters([1, 2, 10, 11, 100]) == [[1, 2], [10, 11], [100]]


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
