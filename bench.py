#!/usr/bin/env python3
"""Paged-KV attention benchmark on one MI355X.

Default run (N = 1):
  * decode: 64 decode tokens, contexts U[512, 4096], one Llama-3-8B-shaped layer
    (Hq 32 / Hkv 8, head dim 128, fp16, 16-token blocks, shuffled arena).  A
    step = the 64 new tokens' append (RoPE, arena write) and the decode, as
    the two boundary calls kv_append_rope + paged_attention_decode (split
    kernel + log-sum-exp combine; drawn queries in, rotated queries to a
    buffer of their own, so every step sees the same input).  `value` is the
    algorithmic decode bytes of one step / step time; `roofline` refers to
    the decode call.  The same step as one paged_attention_decode_append call
    (the append fused into the split kernel, a faster step) is reported beside
    it ("decode_append_fused", with its own roofline); --fused-append makes
    the fused call the timed step and the `roofline` kernel, and reports the
    two-call form as "decode_separate_calls".
  * chunk prefill (reported under "chunk_prefill"): 8 sequences with cached
    prefixes 16*U{0..224} and a 512-token chunk each; a step = kv_append_rope
    + paged_attention_chunk (as its two halves: the plan, then the run);
    TFLOP/s over visible pairs.  The roofline's launch time is the run's
    alone (the attention kernel), over one plan of the batch.
  * decode over INT8 / INT4 arenas ("decode_int8", "decode_int4"): the same
    batch with K/V cached as codes plus one fp16 scale per (token, KV head)
    vector; the chunk workload over the same arenas ("chunk_prefill_int8",
    "chunk_prefill_int4").
  * swap (reported under "swap"): 1024 blocks (64 MiB) of the decode batch out
    to pinned host memory and back (pkv_swap_out / pkv_swap_in), beside a
    plain contiguous copy of the same size in each direction.
Inputs are synthetic and resident in HBM before timing.  Each timed step
rotates over --layers copies of the arena (a layer's worth each) so repeated
steps cannot be served from the 256 MB Infinity Cache.

`roofline` refers to the dominant kernel call (paged_attention_decode): its
average duration over --steps calls issued back to back (rotating the arena
copies) between two HIP events on the stream it is launched on, the median
of three such windows (`avg_launch_ms`); `avg_launch_ms_isolated` is the mean of per-call events in
a separate pass of the same steps (an event record adds a gap to the stream,
so the timed steps carry no events).  `cpu_baseline` times the CPU oracle on
the same decode workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_F16_TFLOPS = 2516.6     # MI355X dense fp16 MFMA
METRIC = "paged-attn decode HBM GB/s + chunk-prefill TFLOP/s, % of MI355X roofline"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_steps(torch, run_step, steps, warmup, run_step_events=None, kernel_events=None):
    """ms per step over ``steps`` plain steps after ``warmup`` untimed ones,
    bracketed by synchronisations.  Then, if given, the same number of steps
    with HIP events around the attention call (instrumentation only: an event
    record adds a gap to the stream, so it stays out of the timed steps) give
    the mean duration of one isolated call."""
    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run_step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_call = None
    if run_step_events is not None:
        kernel_events.clear()
        for i in range(steps):
            run_step_events(i)
        torch.cuda.synchronize()
        ker_ms = [a.elapsed_time(b) for a, b in kernel_events]
        ms_call = sum(ker_ms) / len(ker_ms)
    return (t1 - t0) * 1e3 / steps, ms_call


def time_back_to_back(torch, call, n, windows=3):
    """Average duration of one call over n calls issued back to back between two
    HIP events on the stream the kernels are launched on; the median of
    ``windows`` such windows (the first window after a change of workload can
    still catch the clocks settling)."""
    stream = torch.cuda.current_stream()
    for i in range(3):
        call(i)
    per_call = []
    for _ in range(windows):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            call(i)
        b.record(stream)
        b.synchronize()
        per_call.append(a.elapsed_time(b) / n)
    return sorted(per_call)[len(per_call) // 2]


def make_layers(torch, dw, n):
    layers = [(dw.k_arena, dw.v_arena)]
    for _ in range(n - 1):
        layers.append((dw.k_arena.clone(), dw.v_arena.clone()))
    return layers


def bench_decode(torch, args, kv_bits=0):
    """The decode step on the decode workload, rotating the arena copies.  For
    fp16 arenas the step is one paged_attention_decode_append call (the new
    tokens' append fused into the decode), and the same step as two calls
    (kv_append_rope then paged_attention_decode) and the decode call alone are
    timed beside it (--fused-append swaps the two forms); for quantized
    arenas the step is the two calls, with the fused call timed beside it."""
    import dataclasses
    from paged_kv_chunked_amd import harness, workloads
    w = workloads.decode_batch()
    if kv_bits:
        w = dataclasses.replace(w, kv_bits=kv_bits)
    log(f"decode set-up: {w.num_blocks} blocks")
    dw = harness.DeviceWorkload(w)
    layers = make_layers(torch, dw, args.layers)
    fused = kv_bits == 0 and args.fused_append
    events = []

    def call(i):
        k, v = layers[i % len(layers)]
        if fused:
            dw.decode_append(k_arena=k, v_arena=v)
        else:
            dw.decode(k_arena=k, v_arena=v)

    def run(i):
        if not fused:
            k, v = layers[i % len(layers)]
            dw.append(k_arena=k, v_arena=v)
        call(i)

    def run_events(i):
        if not fused:
            k, v = layers[i % len(layers)]
            dw.append(k_arena=k, v_arena=v)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        call(i)
        b.record()
        events.append((a, b))

    ms_step, ms_call = time_steps(torch, run, args.steps, args.warmup, run_events, events)
    ms_kernel = time_back_to_back(torch, call, args.steps)
    nbytes = dw.decode_append_bytes() if fused else dw.decode_bytes()
    extra = {"fused": fused}
    if kv_bits == 0:
        # the other form of the same step, and the decode call alone
        def sep(i):
            k, v = layers[i % len(layers)]
            dw.append(k_arena=k, v_arena=v)
            dw.decode(k_arena=k, v_arena=v)

        def fus(i):
            k, v = layers[i % len(layers)]
            dw.decode_append(k_arena=k, v_arena=v)

        def dec(i):
            k, v = layers[i % len(layers)]
            dw.decode(k_arena=k, v_arena=v)

        extra["ms_per_step_other_form"] = time_back_to_back(torch, sep if fused else fus,
                                                            args.steps)
        extra["ms_decode_call"] = time_back_to_back(torch, dec, args.steps) if fused else ms_kernel
        extra["decode_append_bytes"] = dw.decode_append_bytes()
    else:
        extra["ms_decode_call"] = ms_kernel

        def fus(i):
            k, v = layers[i % len(layers)]
            dw.decode_append(k_arena=k, v_arena=v)

        extra["ms_per_step_fused_call"] = time_back_to_back(torch, fus, args.steps)
    return w, dw, ms_step, ms_kernel, ms_call, nbytes, extra


def bench_chunk(torch, args, kv_bits=0):
    import dataclasses
    from paged_kv_chunked_amd import harness, workloads
    w = workloads.chunk_batch()
    if kv_bits:
        w = dataclasses.replace(w, kv_bits=kv_bits)
    log(f"chunk set-up: {w.num_blocks} blocks")
    dw = harness.DeviceWorkload(w)
    layers = make_layers(torch, dw, args.layers)
    events = []

    # A step is the append and the attention call as paged_attention_chunk
    # does it: the plan (the schedule) then the run.  The attention kernel's
    # own launch time is that of paged_attention_chunk_run alone, over the
    # plan made once for the batch (a serving step plans once per batch and
    # runs every layer over it).
    def run(i):
        k, v = layers[i % len(layers)]
        dw.append(k_arena=k, v_arena=v)
        dw.chunk_plan()
        dw.chunk_run(k_arena=k, v_arena=v)

    def run_events(i):
        k, v = layers[i % len(layers)]
        dw.append(k_arena=k, v_arena=v)
        dw.chunk_plan()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dw.chunk_run(k_arena=k, v_arena=v)
        b.record()
        events.append((a, b))

    ms_step, ms_call = time_steps(torch, run, args.steps, args.warmup, run_events, events)

    def call(i):
        k, v = layers[i % len(layers)]
        dw.chunk_run(k_arena=k, v_arena=v)

    dw.chunk_plan()
    ms_kernel = time_back_to_back(torch, call, args.steps)

    def whole(i):
        k, v = layers[i % len(layers)]
        dw.chunk(k_arena=k, v_arena=v)

    ms_whole_call = time_back_to_back(torch, whole, args.steps)
    return w, dw, ms_step, ms_kernel, ms_call, dw.chunk_flops(), ms_whole_call


def bench_swap(torch, dw, reps=5):
    """Preemption by swapping: the blocks of the decode batch's longest
    sequences (1024 blocks, 64 MiB) out to pinned host memory and back, against
    a plain contiguous copy of the same size in each direction."""
    import numpy as np
    import paged_kv_chunked_amd as pkv
    order = np.argsort(-dw.dec_lens_host)
    ids = []
    for r in order:
        n = -(-int(dw.dec_lens_host[r]) // 16)
        ids.extend(int(b) for b in dw.bt_host[r, :n])
        if len(ids) >= 1024:
            break
    ids = torch.tensor(ids[:1024], dtype=torch.int32, device=dw.device)
    nbytes = pkv.pkv_swap_bytes(dw.g, ids.shape[0])
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(nbytes, dtype=torch.uint8, device=dw.device)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9

    res = {
        "blocks": int(ids.shape[0]),
        "bytes": nbytes,
        "swap_out_GBps": timed(lambda: pkv.pkv_swap_out(dw.g, dw.k_arena, dw.v_arena, ids, host)),
        "swap_in_GBps": timed(lambda: pkv.pkv_swap_in(dw.g, dw.k_arena, dw.v_arena, ids, host)),
        "copy_d2h_GBps": timed(lambda: host.copy_(dev, non_blocking=True)),
        "copy_h2d_GBps": timed(lambda: dev.copy_(host, non_blocking=True)),
    }
    return {k: (round(v, 2) if isinstance(v, float) else v) for k, v in res.items()}


def bench_shared(torch, args):
    """Decode over a shared prefix: 64 sequences continuing one 4096-token
    prompt, through paged_attention_decode and paged_attention_decode_shared
    (the prompt's whole splits read once per 4 rows)."""
    from paged_kv_chunked_amd import harness, workloads
    w = workloads.shared_prefix_decode()
    log(f"shared-prefix decode set-up: {w.num_blocks} blocks")
    dw = harness.DeviceWorkload(w)
    dw.step()
    ms_plain = time_back_to_back(torch, lambda i: dw.decode(), args.steps)
    ms_shared = time_back_to_back(torch, lambda i: dw.decode_shared(), args.steps)
    nbytes = dw.decode_bytes()
    tokens = int(sum(dw.dec_lens_host))
    res = {
        "workload": "shared_prefix_decode: 64 sequences forked from one 4096-token prompt, "
                    "own tokens U[1,512], Hq 32 / Hkv 8, head_dim 128, fp16",
        "groups": int(len(dw.dec_group_start) - 1),
        "shared_splits": int(dw.dec_max_skip),
        "context_tokens": tokens,
        "unique_bytes": nbytes,
        "ms_decode": round(ms_plain, 5),
        "ms_decode_shared": round(ms_shared, 5),
        "speedup": round(ms_plain / ms_shared, 3),
        "context_tokens_per_s_shared": round(tokens / (ms_shared * 1e-3), 1),
        "unique_GBps_shared": round(nbytes / (ms_shared * 1e-3) / 1e9, 1),
    }
    del dw
    return res


def bench_mixed(torch, args):
    """One continuous-batching step (4 chunks of 256 + 1024 decodes, 16 of them
    sharing a prefix): the separate chunk and decode calls, back to back,
    against one paged_attention_mixed call.  The step's roofline is the sum of
    the decode bytes at HBM peak and the chunk flops at fp16 MFMA peak (no
    credit for overlapping them)."""
    from paged_kv_chunked_amd import harness, workloads
    w = workloads.mixed_step()
    log(f"mixed step set-up: {w.num_blocks} blocks")
    dw = harness.DeviceWorkload(w)
    dw.step()
    dw.mixed()
    n = max(args.steps // 5, 5)
    ms_sep = time_back_to_back(torch, lambda i: (dw.chunk(), dw.decode()), n)
    ms_mix = time_back_to_back(torch, lambda i: dw.mixed(), n)
    # each part of the step as its own call, against its own roofline
    ms_dec = time_back_to_back(torch, lambda i: dw.decode(), n)
    ms_chk = time_back_to_back(torch, lambda i: dw.chunk(), n)
    # the whole step: the 2048 new tokens appended, then the attention
    ms_sep_step = time_back_to_back(torch, lambda i: (dw.append(), dw.chunk(), dw.decode()), n)
    ms_mix_step = time_back_to_back(torch, lambda i: (dw.append(), dw.mixed()), n)
    nbytes, flops = dw.decode_bytes(), dw.chunk_flops()
    roof_ms = (nbytes / (PEAK_HBM_GBS * 1e9) + flops / (PEAK_F16_TFLOPS * 1e12)) * 1e3
    res = {
        "workload": "mixed_step: 4 chunks x 256 rows (P = 16*U{0..496}) + 1024 decodes "
                    "(contexts U[256,8192], 16 sharing a 1024-token prefix), Hq 32 / Hkv 8, "
                    "head_dim 128, fp16",
        "decode_bytes": nbytes,
        "chunk_flops": flops,
        "ms_separate_calls": round(ms_sep, 5),
        "ms_mixed_call": round(ms_mix, 5),
        "speedup": round(ms_sep / ms_mix, 3),
        "ms_step_append_separate_calls": round(ms_sep_step, 5),
        "ms_step_append_mixed_call": round(ms_mix_step, 5),
        "decode_call": {
            "kernel": "paged_attention_decode (decode_split_kernel + decode_combine_kernel<2>)",
            "bound": "hbm", "ms": round(ms_dec, 5), "bytes": nbytes,
            "achieved": round(nbytes / (ms_dec * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / (ms_dec * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        },
        "chunk_call": {
            "kernel": "paged_attention_chunk (chunk_order_kernel + chunk_mfma_kernel<0>, "
                      "keys split into parts + chunk_combine_kernel)",
            "bound": "mfma", "ms": round(ms_chk, 5), "flops": flops,
            "achieved": round(flops / (ms_chk * 1e-3) / 1e12, 2), "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / (ms_chk * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
        },
        "roofline": {
            "kernel": "paged_attention_mixed (mixed_order_kernel + mixed_kernel + "
                      "decode_combine_kernel)",
            "bound": "hbm+mfma",
            "roofline_ms": round(roof_ms, 5),
            "frac": round(roof_ms / ms_mix, 4),
        },
    }
    del dw
    return res


def bench_long(torch, args):
    """The long-context step: 32 decodes at context 32768 and one 4096-token
    chunk at P = 28672 over a 68 750-block arena (4.5 GB per K/V pair of
    arenas, beyond the Infinity Cache by itself), each call against its own
    roofline."""
    from paged_kv_chunked_amd import harness, workloads
    w = workloads.long_context()
    log(f"long-context set-up: {w.num_blocks} blocks")
    dw = harness.DeviceWorkload(w)
    dw.step()
    n = max(args.steps // 5, 5)
    ms_dec = time_back_to_back(torch, lambda i: dw.decode(), n)
    ms_chk = time_back_to_back(torch, lambda i: dw.chunk(), n)
    ms_step = time_back_to_back(torch, lambda i: dw.step(), n)
    nbytes, flops = dw.decode_bytes(), dw.chunk_flops()
    res = {
        "workload": "long_llama3_8b: 32 decodes at 32768 + one 4096-token chunk at P = 28672, "
                    "Hq 32 / Hkv 8, head_dim 128, fp16, 68750-block arena, 1% of keys x8",
        "decode": {"ms": round(ms_dec, 5), "bytes": nbytes,
                   "GBps": round(nbytes / (ms_dec * 1e-3) / 1e9, 1),
                   "frac_hbm": round(nbytes / (ms_dec * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "chunk": {"ms": round(ms_chk, 5), "flops": flops,
                  "TFLOPs": round(flops / (ms_chk * 1e-3) / 1e12, 1),
                  "frac_mfma": round(flops / (ms_chk * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)},
        "ms_step_append_chunk_decode": round(ms_step, 5),
    }
    del dw
    return res


def blas_info():
    """Threads the oracle's BLAS runs with and which BLAS it is."""
    try:
        import threadpoolctl
        pools = threadpoolctl.threadpool_info()
    except Exception:  # pragma: no cover - reporting only
        pools = []
    blas = [p for p in pools if p.get("user_api") == "blas"]
    threads = max((p.get("num_threads", 1) for p in blas), default=1)
    build = ", ".join(f"{p.get('internal_api')} {p.get('version')} "
                      f"({os.path.basename(p.get('filepath', ''))})" for p in blas) or "unknown"
    return threads, build


def bench_tp8(torch, args):
    """One GPU's share of the layer split by KV head over 8 GPUs (Hq 4 / Hkv 1):
    the decode and chunk workloads at that shape, each call against its own
    roofline (decode rotates 4 arena copies; the chunk call splits its 64 row
    tiles' keys into parts)."""
    from paged_kv_chunked_amd import harness, workloads
    res = {"workload": "decode and chunk workloads at Hq 4 / Hkv 1 (one of 8 GPUs splitting "
                       "the Llama-3-8B layer by KV head), head_dim 128, fp16"}
    for kind, w in (("decode", workloads.tp8_decode_batch()), ("chunk", workloads.tp8_chunk_batch())):
        dw = harness.DeviceWorkload(w)
        dw.step()
        layers = make_layers(torch, dw, args.layers)
        if kind == "decode":
            ms = time_back_to_back(torch, lambda i: dw.decode(k_arena=layers[i % len(layers)][0],
                                                              v_arena=layers[i % len(layers)][1]),
                                   args.steps)
            nb = dw.decode_bytes()
            res["decode"] = {"kernel": "paged_attention_decode", "bound": "hbm", "ms": round(ms, 5),
                             "bytes": nb, "achieved": round(nb / (ms * 1e-3) / 1e9, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

            # the whole decode step (the 64 new tokens' append + decode), as two
            # calls and as one paged_attention_decode_append call
            def sep(i):
                k, v = layers[i % len(layers)]
                dw.append(k_arena=k, v_arena=v)
                dw.decode(k_arena=k, v_arena=v)

            def fus(i):
                k, v = layers[i % len(layers)]
                dw.decode_append(k_arena=k, v_arena=v)

            res["decode"]["ms_step_separate_calls"] = round(time_back_to_back(torch, sep, args.steps), 5)
            res["decode"]["ms_step_fused_call"] = round(time_back_to_back(torch, fus, args.steps), 5)
        else:
            ms = time_back_to_back(torch, lambda i: dw.chunk(k_arena=layers[i % len(layers)][0],
                                                             v_arena=layers[i % len(layers)][1]),
                                   args.steps)
            fl = dw.chunk_flops()
            res["chunk"] = {"kernel": "paged_attention_chunk", "bound": "mfma", "ms": round(ms, 5),
                            "flops": fl, "achieved": round(fl / (ms * 1e-3) / 1e12, 2),
                            "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)}
        del dw, layers
    return res


def cpu_baseline(w, target_s, reps=3):
    """The oracle (numpy fp64) on the decode workload: append + attention for
    every decode row, repeated until about target_s / reps seconds have passed;
    the median rate of ``reps`` such runs."""
    from oracle import script as oscript
    from paged_kv_chunked_amd import harness
    st = oscript.run_script(w)
    cu = [0]
    for s in w.step:
        cu.append(cu[-1] + s.count)
    scale = harness.default_scale(w.head_dim)
    runs = []
    for _ in range(reps):
        t0 = time.perf_counter()
        passes = 0
        while True:
            q_rot = oscript.append_step(w, st)
            for r in range(len(w.step)):
                oscript.attend_row(w, st, r, q_rot[cu[r]:cu[r + 1]], scale)
            passes += 1
            if time.perf_counter() - t0 >= target_s / reps:
                break
        runs.append((time.perf_counter() - t0, passes))
    runs.sort(key=lambda x: x[1] / x[0])
    return runs[len(runs) // 2]


def cpu_baseline_chunk(w, target_s, reps=3):
    """The oracle on the chunk workload: the attention of whole chunk
    sequences (512 rows, all heads, fp64 dense masked softmax) taken in step
    order until about target_s / reps seconds have passed; the median rate of
    ``reps`` runs, in visible-pair flops (4 D Hq per pair) per second."""
    from oracle import script as oscript
    from paged_kv_chunked_amd import harness
    st = oscript.run_script(w)
    q_rot = oscript.append_step(w, st)
    cu = [0]
    for s in w.step:
        cu.append(cu[-1] + s.count)
    scale = harness.default_scale(w.head_dim)
    per_pair = 4 * w.head_dim * w.num_q_heads
    runs = []
    for k in range(reps):
        t0 = time.perf_counter()
        flops, seqs = 0, 0
        while True:
            r = (k + seqs) % len(w.step)
            s = w.step[r]
            oscript.attend_row(w, st, r, q_rot[cu[r]:cu[r + 1]], scale)
            flops += per_pair * (s.count * s.start + s.count * (s.count + 1) // 2)
            seqs += 1
            if time.perf_counter() - t0 >= target_s / reps:
                break
        runs.append((time.perf_counter() - t0, flops, seqs))
    runs.sort(key=lambda x: x[1] / x[0])
    return runs[len(runs) // 2]


def plain_rates_GBps(torch, nbytes, copies=4, reps=20):
    """Plain device streams over ``nbytes`` in the same run, as the achievable
    HBM rate beside the decode's: a read (pkv_stream_read: the 16-byte
    non-temporal loads of the decode's K/V reads in a grid-stride loop) and a
    device copy (torch; read + write bytes counted), each over ``copies``
    buffers in turn so repeated passes are not served by the Infinity Cache."""
    import paged_kv_chunked_amd as pkv
    n = nbytes // 16 * 4
    bufs = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(copies)]
    dst = torch.empty(n, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def timed(fn):
        for i in range(copies):
            fn(i)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            fn(i)
        e.record()
        e.synchronize()
        return a.elapsed_time(e) / reps

    ms_read = timed(lambda i: pkv.pkv_stream_read(bufs[i % copies], sink))
    ms_copy = timed(lambda i: dst.copy_(bufs[i % copies]))
    del bufs, dst, sink
    return n * 4 / (ms_read * 1e-3) / 1e9, 2 * n * 4 / (ms_copy * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=4,
                    help="arena copies rotated over (Infinity Cache guard)")
    ap.add_argument("--no-chunk", action="store_true")
    ap.add_argument("--no-swap", action="store_true")
    ap.add_argument("--no-int8", action="store_true")
    ap.add_argument("--no-shared", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-tp8", action="store_true")
    ap.add_argument("--fused-append", action="store_true",
                    help="time the fp16 decode step as one paged_attention_decode_append call")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode leg (profiling the chunk kernel alone)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before timing, copy this many MiB once (a device copy of "
                         "known size to scale HBM counters against)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the hot path is a "
              "single-GPU kernel library; see DESIGN.md for how it would shard.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_chunked_amd as pkv
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pkv.lib()
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.no_decode:
        args.no_cpu_baseline = True
        wc, dwc, ms_cstep, ms_chunk, ms_ccall, flops, _ = bench_chunk(torch, args)
        log(f"chunk: step {ms_cstep:.4f} ms, kernel {ms_chunk:.4f} ms, "
            f"{flops / (ms_chunk * 1e-3) / 1e12:.1f} TFLOP/s kernel")
        return

    from paged_kv_chunked_amd.rocprof_summary import load_traffic
    w, dw, ms_step, ms_dec, ms_dcall, nbytes, dextra = bench_decode(torch, args)
    dec_bytes = dw.decode_bytes()
    value = dec_bytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (ms_dec * 1e-3) / 1e9
    fused = dextra["fused"]
    call_name = "paged_attention_decode_append" if fused else "paged_attention_decode"
    call_kernels = ("decode_split_append_kernel" if fused else "decode_split_kernel") + \
        " + decode_combine_kernel"
    log(f"decode: step {ms_step:.4f} ms, call {ms_dec:.4f} ms, {nbytes / 1e6:.1f} MB "
        f"-> {achieved:.0f} GB/s call, {value:.0f} GB/s step")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode_llama3_8b: 64 sequences x 1 query token, contexts U[512,4096], "
                        "Hq 32 / Hkv 8, head_dim 128, fp16 K/V/Q ~ N(0,1), block 16, "
                        "shuffled arena (total + 10%), step = the new tokens' append and the "
                        "decode" + (" in one paged_attention_decode_append call" if fused else
                                    " as kv_append_rope + paged_attention_decode"),
            "num_seqs": len(w.step),
            "context_tokens": int(sum(dw.dec_lens_host)),
            "arena_blocks": w.num_blocks,
            "layers_rotated": args.layers,
        },
        "roofline": {
            "kernel": f"{call_name} ({call_kernels})",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(TRAFFIC, call_name),
            "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_ms": round(ms_dec, 5),
            "avg_launch_ms_isolated": round(ms_dcall, 5),
        },
    }
    ms_dec_call = dextra["ms_decode_call"]
    ms_other = dextra["ms_per_step_other_form"]
    if fused:
        ach_call = dec_bytes / (ms_dec_call * 1e-3) / 1e9
        out["decode_separate_calls"] = {
            "workload": "the same step as kv_append_rope followed by paged_attention_decode",
            "ms_per_step": round(ms_other, 5),
            "value": round(dec_bytes / (ms_other * 1e-3) / 1e9, 2),
            "decode_call": {
                "kernel": "paged_attention_decode (decode_split_kernel + decode_combine_kernel)",
                "bound": "hbm", "ms": round(ms_dec_call, 5), "bytes": dec_bytes,
                "achieved": round(ach_call, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach_call / PEAK_HBM_GBS, 4),
                "traffic": load_traffic(TRAFFIC, "paged_attention_decode"),
            },
        }
    else:
        # the fused form, back to back: its step is the one call
        fb = dextra["decode_append_bytes"]
        ach_f = fb / (ms_other * 1e-3) / 1e9
        out["decode_append_fused"] = {
            "workload": "the same step as one paged_attention_decode_append call (the new "
                        "tokens' RoPE and arena append fused into the split kernel)",
            "ms_per_step": round(ms_other, 5),
            "value": round(dec_bytes / (ms_other * 1e-3) / 1e9, 2),
            "call": {
                "kernel": "paged_attention_decode_append (decode_split_append_kernel + "
                          "decode_combine_kernel)",
                "bound": "hbm", "ms": round(ms_other, 5), "bytes": fb,
                "achieved": round(ach_f, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach_f / PEAK_HBM_GBS, 4),
                "traffic": load_traffic(TRAFFIC, "paged_attention_decode_append"),
            },
        }
    log(f"other form of the step: {ms_other:.4f} ms")
    read_gbs, copy_gbs = plain_rates_GBps(torch, dec_bytes)
    out["roofline"]["plain_read_GBps"] = round(read_gbs, 1)
    out["roofline"]["plain_copy_GBps"] = round(copy_gbs, 1)
    out["roofline"]["frac_of_plain_stream"] = round(achieved / max(read_gbs, copy_gbs), 4)
    log(f"plain device streams of {dec_bytes / 1e6:.1f} MB: read {read_gbs:.0f} GB/s, "
        f"copy {copy_gbs:.0f} GB/s (read + write)")
    if not args.no_swap:
        out["swap"] = bench_swap(torch, dw)
        log(f"swap: {out['swap']}")
    for bits in (() if args.no_int8 else (8, 4)):
        _, dwq, ms_stepq, ms_decq, ms_dcallq, nbytesq, qextra = bench_decode(torch, args,
                                                                            kv_bits=bits)
        achq = nbytesq / (ms_decq * 1e-3) / 1e9
        tokens = int(sum(dwq.dec_lens_host))
        log(f"decode int{bits}: kernel {ms_decq:.4f} ms, {nbytesq / 1e6:.1f} MB -> {achq:.0f} GB/s")
        out[f"decode_int{bits}"] = {
            "workload": f"the decode workload over INT{bits} arenas (codes + one fp16 scale per "
                        "(token, KV head) vector)",
            "context_tokens_per_s": round(tokens / (ms_decq * 1e-3), 1),
            "speedup_vs_fp16_arena": round(ms_dec_call / ms_decq, 3),
            "ms_per_step": round(ms_stepq, 5),
            "ms_per_step_fused_call": round(qextra["ms_per_step_fused_call"], 5),
            "roofline": {
                "kernel": f"paged_attention_decode (decode_split_i{bits}_kernel + "
                          "decode_combine_kernel)",
                "bound": "hbm",
                "achieved": round(achq, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(achq / PEAK_HBM_GBS, 4),
                "traffic": load_traffic(TRAFFIC, f"paged_attention_decode_i{bits}"),
                "algorithmic_bytes_per_launch": nbytesq,
                "avg_launch_ms": round(ms_decq, 5),
                "avg_launch_ms_isolated": round(ms_dcallq, 5),
            },
        }
        del dwq
        # the achievable read rate for this call's byte count, same run
        read_q, _ = plain_rates_GBps(torch, nbytesq)
        out[f"decode_int{bits}"]["roofline"]["plain_read_GBps"] = round(read_q, 1)
        out[f"decode_int{bits}"]["roofline"]["frac_of_plain_read"] = round(achq / read_q, 4)
    if not args.no_shared:
        out["decode_shared_prefix"] = bench_shared(torch, args)
        log(f"shared-prefix decode: {out['decode_shared_prefix']}")
    if not args.no_mixed:
        out["mixed_step"] = bench_mixed(torch, args)
        log(f"mixed step: {out['mixed_step']}")
    if not args.no_long:
        out["long_context"] = bench_long(torch, args)
        log(f"long context: {out['long_context']}")
    if not args.no_tp8:
        out["tp8_shard"] = bench_tp8(torch, args)
        log(f"tp8 shard: {out['tp8_shard']}")
    if not args.no_chunk:
        wc, dwc, ms_cstep, ms_chunk, ms_ccall, flops, ms_cwhole = bench_chunk(torch, args)
        tf_kernel = flops / (ms_chunk * 1e-3) / 1e12
        tf_step = flops / (ms_cstep * 1e-3) / 1e12
        log(f"chunk: step {ms_cstep:.4f} ms, kernel {ms_chunk:.4f} ms, {flops / 1e9:.1f} GFLOP "
            f"-> {tf_kernel:.1f} TFLOP/s kernel")
        out["chunk_prefill"] = {
            "workload": "chunk_llama3_8b: 8 sequences, prefix 16*U{0..224}, 512-token chunk, "
                        "Hq 32 / Hkv 8, head_dim 128, fp16, RoPE theta 5e5",
            "value": round(tf_step, 2),
            "unit": "TFLOP/s",
            "ms_per_step": round(ms_cstep, 5),
            "roofline": {
                "kernel": "paged_attention_chunk_run (chunk_mfma_kernel)",
                "bound": "mfma",
                "achieved": round(tf_kernel, 2),
                "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(tf_kernel / PEAK_F16_TFLOPS, 4),
                "traffic": load_traffic(TRAFFIC, "paged_attention_chunk"),
                "algorithmic_flops_per_launch": flops,
                "avg_launch_ms": round(ms_chunk, 5),
                "avg_launch_ms_isolated": round(ms_ccall, 5),
            },
            "ms_call_with_plan": round(ms_cwhole, 5),
        }
        del dwc
        for bits in (() if args.no_int8 else (8, 4)):
            _, dwq, ms_cstepq, ms_chunkq, ms_ccallq, flopsq, ms_cwholeq = bench_chunk(
                torch, args, kv_bits=bits)
            tfq = flopsq / (ms_chunkq * 1e-3) / 1e12
            log(f"chunk int{bits}: kernel {ms_chunkq:.4f} ms -> {tfq:.1f} TFLOP/s")
            out[f"chunk_prefill_int{bits}"] = {
                "workload": f"the chunk workload over INT{bits} arenas, dequantized to fp16 "
                            "tiles in LDS",
                "ms_per_step": round(ms_cstepq, 5),
                "speedup_vs_fp16_arena": round(ms_chunk / ms_chunkq, 3),
                "roofline": {
                    "kernel": f"paged_attention_chunk_run (chunk_mfma_kernel<{1 if bits == 8 else 2}>)",
                    "bound": "mfma",
                    "achieved": round(tfq, 2),
                    "peak": PEAK_F16_TFLOPS,
                    "unit": "TFLOP/s",
                    "frac": round(tfq / PEAK_F16_TFLOPS, 4),
                    "traffic": load_traffic(TRAFFIC, f"paged_attention_chunk_i{bits}"),
                    "algorithmic_flops_per_launch": flopsq,
                    "avg_launch_ms": round(ms_chunkq, 5),
                    "avg_launch_ms_isolated": round(ms_ccallq, 5),
                },
                "ms_call_with_plan": round(ms_cwholeq, 5),
            }
            del dwq
    out["library_source_hash"] = pkv.pkv_source_hash()
    if not args.no_cpu_baseline:
        threads, build = blas_info()
        affinity = len(os.sched_getaffinity(0))
        log("cpu baseline (oracle), decode workload")
        secs, passes = cpu_baseline(w, args.cpu_seconds)
        out["cpu_baseline"] = {
            "value": round(nbytes * passes / secs / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"the whole decode step (append + attention, {len(w.step)} sequences) "
                      f"x {passes} passes in {secs:.1f} s (median of 3 runs), numpy fp64",
            "host_cores_available": affinity,
            "blas": build,
        }
        if "chunk_prefill" in out:
            from paged_kv_chunked_amd import workloads
            log("cpu baseline (oracle), chunk workload")
            secs, flops, seqs = cpu_baseline_chunk(workloads.chunk_batch(), args.cpu_seconds)
            out["chunk_prefill"]["cpu_baseline"] = {
                "value": round(flops / secs / 1e12, 6),
                "unit": "TFLOP/s",
                "cores": threads,
                "kind": "oracle",
                "sample": f"{seqs} of the 8 chunk sequences' attention (512 rows x 32 heads "
                          f"each) in {secs:.1f} s (median of 3 runs), numpy fp64",
                "host_cores_available": affinity,
                "blas": build,
            }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
