"""Summaries of rocprofv3 result databases for profiles/.

    python -m paged_kv_chunked_amd.rocprof_summary stats DB OUT.md --command "..." [--note ...]
        dispatch count and average / min / max / total duration per (kernel,
        grid) (a --kernel-trace --stats run).
    python -m paged_kv_chunked_amd.rocprof_summary counters DB OUT.json --kernel NAME ... \
            --command "..." [--simds 1024] [--flops F]
        per-dispatch averages of the counters of a --pmc run for the named
        kernels, with MFMA busy % and MFMA flops where those counters exist.
    python -m paged_kv_chunked_amd.rocprof_summary traffic FETCH_DB WRITE_DB OUT.json \
            --copy-mib N --command "..."
        HBM bytes per dispatch from two --pmc runs (FETCH_SIZE, then WRITE_SIZE).
        Each counter is scaled by what it reads for the device copy of N MiB
        that bench.py --calibrate-copy-mib N performs first (the first
        __amd_rocclr_copyBuffer dispatch): scale = N MiB / counter value.  The
        record stores the SHA-256 of the kernel sources, so bench.py only uses
        it while those sources are unchanged.  Dispatches are averaged per
        kernel name, so the profiled command must run each kernel on one
        workload only (bench.py --no-shared --no-swap --no-mixed).

rocprofv3 writes one SQLite database per process; its ``kernels`` and
``pmc_events`` views are read here.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import sqlite3

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernel call -> (kernel symbol substrings, source files whose change invalidates it)
_DECODE_SRC = ("decode.hip", "decode_core.h", "decode_q_core.h", "fp16_shape.h", "lds_dma.h",
               "pkv_internal.h", "quant_codes.h", "quant_append_core.h", "rope_core.h")
_CHUNK_SRC = ("chunk.hip", "chunk_core.h", "fp16_shape.h", "lds_dma.h", "pkv_internal.h",
              "quant_codes.h")
CALLS = {
    "paged_attention_decode": (("decode_split_kernel", "decode_combine_kernel"), _DECODE_SRC),
    "paged_attention_decode_append": (("decode_split_append_kernel", "decode_combine_kernel"),
                                      _DECODE_SRC),
    "paged_attention_decode_i8": (("decode_split_i8_kernel", "decode_combine_kernel"),
                                  _DECODE_SRC),
    "paged_attention_decode_i4": (("decode_split_i4_kernel", "decode_combine_kernel"),
                                  _DECODE_SRC),
    # chunk_mfma_kernel<kQ>: fp16 (0), INT8 (1), INT4 (2) arenas (the trace
    # holds the mangled or the demangled name; one of the two matches)
    "paged_attention_chunk": (("chunk_mfma_kernelILi0E", "chunk_mfma_kernel<0>"),
                                  _CHUNK_SRC),
    "paged_attention_chunk_i8": (("chunk_mfma_kernelILi1E", "chunk_mfma_kernel<1>"),
                                  _CHUNK_SRC),
    "paged_attention_chunk_i4": (("chunk_mfma_kernelILi2E", "chunk_mfma_kernel<2>"),
                                  _CHUNK_SRC),
    "paged_attention_mixed": (("mixed_kernel", "mixed_order_kernel"),
                              ("mixed.hip", "chunk_core.h", "decode_core.h", "decode_q_core.h",
                               "fp16_shape.h", "lds_dma.h", "pkv_internal.h", "quant_codes.h",
                               "quant_append_core.h", "rope_core.h")),
    "kv_append_rope": (("append_rope_kernel", "append_rope_vec_kernel", "append_rope_block_kernel"),
                       ("append.hip", "rope_core.h", "quant_append_core.h", "pkv_internal.h")),
}


def sources_sha(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_rows(db):
    c = sqlite3.connect(db)
    return c.execute("select name, grid_x, grid_y, grid_z, duration from kernels").fetchall()


def split_clusters(durs, ratio=1.5):
    """Durations of one (kernel, grid) cut at every gap where the next-longer
    launch takes more than ``ratio`` times as long: two workloads that happen
    to launch the same grid (a short and a long one) get separate lines.  The
    launches of one workload spread less than that (under 1.3x here)."""
    durs = sorted(durs)
    groups, cur = [], [durs[0]]
    for a, b in zip(durs, durs[1:]):
        if b > ratio * a:
            groups.append(cur)
            cur = []
        cur.append(b)
    return groups + [cur]


def stats_rows(rows, min_calls=5):
    """(kernel, grid) -> launch durations, from (name, gx, gy, gz, duration)
    rows.  Launches of one kernel on different workloads have different grids
    and are kept apart; a (kernel, grid) whose durations fall into clusters
    more than 1.5x apart is listed once per cluster (grid marked #1, #2, ...
    from the shortest).  Grids with fewer than min_calls launches (set-up work
    such as cache fills of varying size) are folded into one row per kernel,
    "other grids (n)"."""
    raw = collections.defaultdict(list)
    for name, gx, gy, gz, dur in rows:
        raw[(name, f"{gx}x{gy}x{gz}")].append(dur)
    agg, rest = {}, collections.defaultdict(list)
    nrest = collections.Counter()
    for (name, grid), durs in raw.items():
        if len(durs) < min_calls:
            rest[name] += durs
            nrest[name] += 1
            continue
        groups = split_clusters(durs)
        for i, grp in enumerate(groups):
            agg[(name, grid if len(groups) == 1 else f"{grid} #{i + 1}")] = grp
    for name, durs in rest.items():
        agg[(name, f"other grids ({nrest[name]})")] = durs
    return agg


def stats(db, out, command, notes=()):
    """The kernel statistics table of a kernel trace (rows as stats_rows)."""
    agg = stats_rows(kernel_rows(db))
    lines = [f"# rocprofv3 kernel statistics", "", f"Command: `{command}`", ""]
    lines += [f"- {n}" for n in notes] + ([""] if notes else [])
    lines += ["| kernel | grid (threads) | calls | avg (us) | min (us) | max (us) | total (ms) |",
              "|---|---|---|---|---|---|---|"]
    for (name, grid), durs in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) < 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {grid} | {len(durs)} | {sum(durs) / len(durs) / 1e3:.2f} | "
                     f"{min(durs) / 1e3:.2f} | {max(durs) / 1e3:.2f} | {sum(durs) / 1e6:.3f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _pmc(db, counter):
    c = sqlite3.connect(db)
    rows = c.execute("select dispatch_id, name, counter_value from pmc_events "
                     "where counter_name = ? order by dispatch_id", (counter,)).fetchall()
    return rows


def traffic(fetch_db, write_db, out, copy_mib, command):
    copy_kib = copy_mib * 1024.0
    rec = {"command": command, "copy_mib": copy_mib, "calls": {}}
    for key, db, counter in (("fetch", fetch_db, "FETCH_SIZE"), ("write", write_db, "WRITE_SIZE")):
        rows = _pmc(db, counter)
        copy = [v for _, n, v in rows if "copyBuffer" in n]
        scale = copy_kib / copy[0]
        rec[f"{key}_scale"] = scale
        for call, (syms, _) in CALLS.items():
            per = collections.defaultdict(list)
            for _, name, v in rows:
                for sname in syms:
                    if sname in name:
                        per[sname].append(v)
            if not per:
                continue
            entry = rec["calls"].setdefault(call, {})
            kib = sum(sum(v) / len(v) for v in per.values())
            entry[f"{key}_kib_per_call_raw"] = kib
            entry[f"{key}_bytes_per_call"] = kib * scale * 1024.0
            entry["kernels"] = sorted(per)
    for call, (_, files) in CALLS.items():
        if call in rec["calls"]:
            rec["calls"][call]["sources_sha256"] = sources_sha(files)
            rec["calls"][call]["sources"] = list(files)
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)


def counters(db, out, command, kernels, simds, flops=None, notes=()):
    """Per-dispatch averages of every counter of a --pmc run for each kernel
    whose name contains one of ``kernels`` (dispatches on different grids, or
    in duration clusters more than 1.5x apart, listed apart), with the
    kernel-trace duration of the same dispatches, and where the counters are
    present:
      mfma_busy_pct = sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES
                      / (max over XCDs of GRBM_GUI_ACTIVE * simds) * 100
      mfma_f16_flop = SQ_INSTS_VALU_MFMA_MOPS_F16 * 512 (products issued,
                      masked work included), and its ratio to the algorithmic
                      flops of one dispatch: ``flops`` maps a row's grid label
                      (e.g. "262144x1x1 #1") to them.
    """
    flops = flops or {}
    c = sqlite3.connect(db)
    disp = {}
    for did, name, gx, gy, gz, dur in c.execute(
            "select dispatch_id, name, grid_x, grid_y, grid_z, duration from kernels"):
        disp[did] = (name, f"{gx}x{gy}x{gz}", dur)
    # one row per hardware instance: SQ counters come per shader engine and are
    # summed; GRBM counters come per XCD, each counting the same active
    # cycles, and are reduced by their maximum
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    for did, name, cname, v in c.execute(
            "select dispatch_id, name, counter_name, counter_value from pmc_events"):
        if cname.startswith("GRBM_"):
            vals[did][cname] = max(vals[did][cname], v)
        else:
            vals[did][cname] += v
    groups = collections.defaultdict(list)
    for did, cv in vals.items():
        name, grid, dur = disp.get(did, (None, None, None))
        if name is None or not any(k in name for k in kernels):
            continue
        groups[(name, grid)].append((dur, cv))
    split = {}
    for (name, grid), rows in groups.items():
        clusters = split_clusters([d for d, _ in rows])
        for i, cl in enumerate(clusters):
            lo, hi = cl[0], cl[-1]
            split[(name, grid if len(clusters) == 1 else f"{grid} #{i + 1}")] = [
                r for r in rows if lo <= r[0] <= hi]
    rec = {"command": command, "simds": simds, "notes": list(notes), "kernels": []}
    for (name, grid), rows in sorted(split.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        n = len(rows)
        avg = collections.defaultdict(float)
        for _, cv in rows:
            for k, v in cv.items():
                avg[k] += v / n
        entry = {"kernel": name, "grid": grid, "dispatches": n,
                 "avg_duration_us": sum(d for d, _ in rows) / n / 1e3,
                 "counters_per_dispatch": dict(sorted(avg.items()))}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg.get("GRBM_GUI_ACTIVE"):
            entry["mfma_busy_pct"] = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (
                avg["GRBM_GUI_ACTIVE"] * simds)
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in avg:
            entry["mfma_f16_flop"] = avg["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512.0
            if grid in flops:
                entry["algorithmic_flop"] = flops[grid]
                entry["mfma_f16_flop_over_algorithmic"] = entry["mfma_f16_flop"] / flops[grid]
        rec["kernels"].append(entry)
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def load_traffic(path, call):
    """Bytes per call (fetch + write) if the record matches the current sources."""
    try:
        with open(path) as fh:
            rec = json.load(fh)
        entry = rec["calls"][call]
        if entry["sources_sha256"] != sources_sha(entry["sources"]):
            return None
        return entry["fetch_bytes_per_call"] + entry["write_bytes_per_call"]
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("counters")
    a.add_argument("db")
    a.add_argument("out")
    a.add_argument("--command", required=True)
    a.add_argument("--kernel", action="append", required=True)
    a.add_argument("--simds", type=int, default=1024)
    a.add_argument("--flops", action="append", default=[],
                   help="GRID_LABEL=FLOPS, algorithmic flops of one dispatch of that row")
    a.add_argument("--note", action="append", default=[])
    a = sub.add_parser("stats")
    a.add_argument("db")
    a.add_argument("out")
    a.add_argument("--command", required=True)
    a.add_argument("--note", action="append", default=[])
    b = sub.add_parser("traffic")
    b.add_argument("fetch_db")
    b.add_argument("write_db")
    b.add_argument("out")
    b.add_argument("--copy-mib", type=int, required=True)
    b.add_argument("--command", required=True)
    args = ap.parse_args()
    if args.cmd == "stats":
        stats(args.db, args.out, args.command, args.note)
    elif args.cmd == "counters":
        fl = {}
        for item in args.flops:
            label, _, val = item.rpartition("=")
            fl[label] = float(val)
        counters(args.db, args.out, args.command, args.kernel, args.simds, fl, args.note)
    else:
        traffic(args.fetch_db, args.write_db, args.out, args.copy_mib, args.command)


if __name__ == "__main__":
    main()
