"""Benchmark of the paged KV-cache hot path on one MI355X.

One step = the whole path over one batch: each sequence's new token is
stored into its slot and attended together with its full paged context, as
one pa_decode_append launch (pa_store_kv + pa_decode is timed beside it).  The
default workload is the largest decode configuration that fits one GPU:
8 sequences of 131,072 cached tokens each (512 blocks per sequence), 32 query
/ 8 kv heads, head dim 128, 256-token blocks, physical blocks shuffled, pool
+10 %: 4.29 GB of K/V read per step.  Inputs are seeded synthetic data placed
in HBM before timing.  The other decode shapes, the prefill and the next-step
workloads are reported under "extra", each with its own roofline object.

Prints ONE JSON line.  `--gpus N` with N > 1 exits: the library and its
benchmark run on one GPU.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import paged_kv_cache_237_amd as pa  # noqa: E402
import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attention: HBM GB/s (% of peak) + attended tokens/sec; prefill TFLOP/s"


def decode_bytes(case: wl.PagedCase) -> int:
    """Algorithmic bytes of one pa_decode: every cached K and V row of every
    context once, q in, out written, block-table entries used, lengths."""
    sum_ctx = int(case.context_lens.sum())
    d, hkv, hq, b = case.head_dim, case.num_kv_heads, case.num_q_heads, case.batch
    blocks = sum(wl.blocks_for(int(n)) for n in case.context_lens)
    return sum_ctx * hkv * d * 2 * 2 + 2 * b * hq * d * 2 + 4 * blocks + 4 * b


def store_bytes(n_tokens: int, hkv: int, d: int = 128) -> int:
    """Algorithmic bytes of one pa_store_kv: K and V rows read and written, slots read."""
    return 2 * n_tokens * hkv * d * 2 * 2 + 4 * n_tokens


def append_bytes(case: wl.PagedCase) -> int:
    """Algorithmic bytes of one pa_decode_append: those of pa_decode (the new
    token's K and V rows come from k_new / v_new instead of the cache, the
    same bytes) plus the new rows written into the cache."""
    n_new = int((case.context_lens > 0).sum())
    return decode_bytes(case) + n_new * case.num_kv_heads * case.head_dim * 2 * 2


def place(case):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from device_case import place as _place  # noqa: E402
    return _place(case)


def copy_probe(mib: int) -> None:
    """One plain device-to-device copy of `mib` MiB (outside any timing)."""
    if mib <= 0:
        return
    src = torch.ones(mib * 2**20 // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_237_amd", "libpa_probe.so")


def read_ceiling(sizes, labels, steps: int = 30) -> dict:
    """Measured HBM read rate of a load-only kernel shaped like the decode
    launch (one 8-wave workgroup per CU, each wave streaming contiguous 32 KiB
    pieces; csrc/read_ceiling.hip), for each byte count in `sizes` (rounded
    down to 32 KiB): what a launch of that shape and size can stream on this
    machine, reported beside the vendor peak -- with the default cache policy
    and with the non-temporal one the decode kernels use ("nt").  None if the
    probe library is not built."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.pa_probe_stream_read.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sizes = [int(n) // 32768 * 32768 for n in sizes]
    buf = torch.zeros(max(sizes), dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {"kernel": "stream_read_kernel (load-only, decode launch shape)", "workgroups": cus}
    for n, label in zip(sizes, labels):
        for nt in (0, 1):
            def call():
                st = lib.pa_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), n, cus, nt,
                                              ctypes.c_void_p(sink.data_ptr()),
                                              ctypes.c_void_p(stream.cuda_stream))
                if st != 0:
                    raise RuntimeError(f"pa_probe_stream_read returned {st}")
            _warm(call, 20)
            ms = _events_batch_ms(call, steps)
            res[label + ("_nt" if nt else "")] = {"bytes": n, "us": round(ms * 1e3, 2),
                                                  "GBps": round(n / (ms * 1e-3) / 1e9, 1)}
    del buf, sink
    torch.cuda.empty_cache()
    return res


def new_rows(dev):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from device_case import new_rows as _new_rows  # noqa: E402
    return _new_rows(dev)


def _graph_of(fn):
    """fn captured once in a HIP graph (after a warm-up call on the capture
    stream)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


def _warm(fn, warmup: int, min_s: float = 0.2) -> None:
    """Calls fn at least `warmup` times and for at least min_s seconds of
    sustained GPU work.  The compute clock ramps up over the first ~50 ms of
    sustained matrix work (prefill calls run ~180 us at first and ~160 us
    after that; after two idle seconds the ramp starts over), so a warm-up
    of a few calls would time the ramp, not the kernel.  Memory-bound decode
    runs at its steady time from the first call."""
    n = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _events_ms(fn, steps, before=None):
    """Mean and list of HIP-event times (ms) of `steps` eager calls of fn, on
    the stream the kernels run on; `before` runs outside the events."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        if before is not None:
            before()
        a.record(torch.cuda.current_stream())
        fn()
        b.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return float(np.mean(ts)), ts


def _events_batch_ms(fn, steps):
    """Mean time (ms) of one call of fn from a pair of HIP events around
    `steps` calls launched back to back on the stream the kernels run on: the
    kernels' own duration plus the few-microsecond gap between two kernels of
    one stream, without the host's launch latency that events around a single
    call also catch."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(torch.cuda.current_stream())
    for _ in range(steps):
        fn()
    b.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_decode(case: wl.PagedCase, steps: int, warmup: int) -> dict:
    """Times `steps` decode steps after `warmup`.  A step stores each
    sequence's new token and attends over the whole context; it runs as one
    pa_decode_append launch ("step_ms", the headline) and, for comparison, as
    pa_store_kv + pa_decode ("two_call_step_ms").  Whole steps are launched
    back to back on one stream (the host stays far ahead of a step of this
    size, so the GPU sees no launch gaps); their HIP-graph replays are timed
    apart (time_decode_graphs), after every single-stream measurement.  Kernel
    times ("append_ms", "decode_ms", "store_ms") are HIP events around
    `steps` eager calls launched back to back on the stream the kernels run
    on, divided by `steps`; "decode_ms_flushed" are
    pa_decode times with the caches (4 MB L2 per XCD, 256 MB MALL) flushed
    before each call by reading 1 GiB of other data, outside the events: what
    one layer of a deep model sees, since its cache is read again only after
    every other layer's (a read leaves clean lines; a write-based flush would
    also charge the decode with writing back 256 MB of dirty lines).  Every
    call writes the same token bytes to the same slots, so the cache state is
    the same for all of them."""
    dev = place(case)
    k_new, v_new = new_rows(dev)
    out = torch.empty((case.batch, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    ws = pa.alloc_decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads)

    def store():
        pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)

    def decode():
        pa.decode(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens,
                  case.max_context_len, case.scale, ws)

    def append():
        pa.decode_append(out, dev.q, k_new, v_new, dev.k_cache, dev.v_cache, dev.block_table,
                         dev.context_lens, case.max_context_len, case.scale, ws)

    def two_calls():
        store()
        decode()

    for _ in range(warmup):
        two_calls()
        append()
    res = {}
    res["append_ms"] = _events_batch_ms(append, steps)
    res["store_ms"] = _events_batch_ms(store, steps)
    res["decode_ms"] = _events_batch_ms(decode, steps)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    _, res["decode_ms_flushed"] = _events_ms(decode, steps,
                                             before=lambda: torch.amax(flush, dim=0, out=sink))
    del flush, sink

    def whole(run):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    res["two_call_step_ms"] = whole(two_calls)
    res["step_ms"] = whole(append)
    del dev
    torch.cuda.empty_cache()
    return res


def time_decode_graphs(case: wl.PagedCase, steps: int, warmup: int) -> dict:
    """The steps of time_decode captured once each in a HIP graph and replayed
    back to back ("step_graph_ms", "two_call_step_graph_ms"; a replay of a
    graph this small adds a few microseconds of its own).  The capture runs
    on a stream of its own, and after a process moves its work between
    streams the kernels that follow can run ~3 % slower (an 8 x 128K decode
    step 636-641 -> 653-660 us per launch, not after every switch), so
    main() times the graphs, and the two-stream forms of the mixed batch,
    after everything else."""
    dev = place(case)
    k_new, v_new = new_rows(dev)
    out = torch.empty((case.batch, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    ws = pa.alloc_decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads)

    def append():
        pa.decode_append(out, dev.q, k_new, v_new, dev.k_cache, dev.v_cache, dev.block_table,
                         dev.context_lens, case.max_context_len, case.scale, ws)

    def two_calls():
        pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
        pa.decode(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens,
                  case.max_context_len, case.scale, ws)

    def whole(run):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    g2, g1 = _graph_of(two_calls), _graph_of(append)
    res = {"two_call_step_graph_ms": whole(g2.replay), "step_graph_ms": whole(g1.replay)}
    del g1, g2, dev
    torch.cuda.empty_cache()
    return res


def prefill_bytes(case: wl.PagedCase) -> int:
    """Algorithmic bytes of one pa_prefill: q in and out written, every
    cached K and V row of every context once, block-table entries used,
    lengths and query offsets."""
    rows = int(case.q_lens.sum())
    sum_ctx = int(case.context_lens.sum())
    d, hkv, hq, b = case.head_dim, case.num_kv_heads, case.num_q_heads, case.batch
    blocks = sum(wl.blocks_for(int(n)) for n in case.context_lens)
    return 2 * rows * hq * d * 2 + sum_ctx * hkv * d * 2 * 2 + 4 * blocks + 4 * b + 4 * (b + 1)


def prefill_flops(case: wl.PagedCase) -> int:
    """Causal FLOPs of one pa_prefill: 4*D per (query row, visible key) pair
    per query head (q.k and p.v, a multiply and an add each)."""
    pairs = 0
    for b in range(case.batch):
        ql, n = int(case.q_lens[b]), int(case.context_lens[b])
        first = n - ql + 1  # keys seen by the first query row
        pairs += ql * first + ql * (ql - 1) // 2
    return 4 * case.head_dim * case.num_q_heads * pairs


PREFILL_SPREAD = {}


def time_prefill(case: wl.PagedCase, steps: int, warmup: int):
    """Times store (all prompt tokens) + prefill, `steps` calls after the
    warm-up; returns the medians (store_ms, prefill_ms) and records the
    prefill min / max in PREFILL_SPREAD."""
    dev = place(case)
    out = torch.empty((case.total_q_rows, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    stream = torch.cuda.current_stream()
    ws = pa.alloc_prefill_workspace(case.batch, case.total_q_rows, case.max_q_len, case.num_q_heads,
                                    case.num_kv_heads, case.max_blocks_per_seq)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
        if ev is not None:
            ev[1].record(stream)
        pa.prefill(out, dev.q, dev.cu_q, dev.context_lens, case.max_q_len, dev.k_cache,
                   dev.v_cache, dev.block_table, case.scale, ws)
        if ev is not None:
            ev[2].record(stream)

    _warm(step, warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    # medians of the per-call times (min and max in PREFILL_SPREAD)
    sts = [e[0].elapsed_time(e[1]) for e in evs]
    pts = [e[1].elapsed_time(e[2]) for e in evs]
    sto, pre = float(np.median(sts)), float(np.median(pts))
    PREFILL_SPREAD[case.name] = {"prefill_ms_min": round(min(pts), 4), "prefill_ms_max": round(max(pts), 4),
                                 "reps": len(pts)}
    del dev
    torch.cuda.empty_cache()
    return sto, pre


def prefill_report(steps: int, warmup: int) -> dict:
    c = wl.prefill_8x2048()
    sto, pre = time_prefill(c, steps, warmup)
    fl = prefill_flops(c)
    sb = store_bytes(c.total_kv_rows, c.num_kv_heads)
    pb = prefill_bytes(c)
    tf = fl / (pre * 1e-3) / 1e12
    return {"workload": c.name, "prefill_ms": round(pre, 4), **PREFILL_SPREAD.get(c.name, {}),
            "causal_gflop": round(fl / 1e9, 3),
            "prefill_TFLOPs": round(tf, 1), "frac_of_bf16_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
            "store_ms": round(sto, 4), "store_tokens": c.total_kv_rows,
            "store_GBps": round(sb / (sto * 1e-3) / 1e9, 1),
            "store_frac_of_hbm_peak": round(sb / (sto * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "store_algorithmic_bytes": sb, "store_traffic_bytes": recorded_store_traffic(),
            "rocprof_counters": recorded_prefill_counters(),
            # the same schema as the headline's roofline, for the prefill and
            # store kernels of this workload
            "prefill_roofline": {"bound": "mfma", "kernel": "prefill_kernel<2>",
                                 "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                 "traffic": recorded_prefill_traffic(), "algorithmic_flops_per_launch": fl,
                                 "algorithmic_bytes_per_launch": pb},
            "store_roofline": {"bound": "hbm", "kernel": "store_kv_kernel",
                               "achieved": round(sb / (sto * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s",
                               "frac": round(sb / (sto * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "traffic": recorded_store_traffic(),
                               "algorithmic_bytes_per_launch": sb}}


def varlen_report(name: str, steps: int, warmup: int) -> dict:
    """pa_prefill on a varlen batch whose rows see long cached contexts
    (chunked prefill mixed with decode rows; multi-query decode): reported
    against both rooflines -- causal FLOPs over the bf16 MFMA peak, and the
    K/V bytes of every context read once over the HBM peak."""
    c = wl.CONFIGS[name]()
    sto, pre = time_prefill(c, steps, warmup)
    fl = prefill_flops(c)
    kvb = int(c.context_lens.sum()) * c.num_kv_heads * c.head_dim * 2 * 2
    tf = fl / (pre * 1e-3) / 1e12
    gbs = kvb / (pre * 1e-3) / 1e9
    fm, fh = tf / BF16_MFMA_PEAK_TFLOPS, gbs / HBM_PEAK_GBS
    # the roofline object names the side the batch is closer to (a batch of
    # short rows reads K/V; one of long chunks computes)
    roof = ({"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(tf, 1),
             "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(fm, 4),
             "algorithmic_flops_per_launch": fl} if fm >= fh else
            {"bound": "hbm", "kernel": "prefill_kernel", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(fh, 4), "algorithmic_kv_bytes_per_launch": kvb})
    roof["traffic"] = None
    return {"workload": c.name, "prefill_ms": round(pre, 4), **PREFILL_SPREAD.get(c.name, {}),
            "query_rows": c.total_q_rows,
            "sum_context_len": int(c.context_lens.sum()), "causal_gflop": round(fl / 1e9, 3),
            "TFLOPs": round(tf, 1), "frac_of_bf16_mfma_peak": round(fm, 4),
            "kv_GBps": round(gbs, 1), "frac_of_hbm_peak": round(fh, 4),
            "store_ms": round(sto, 4), "roofline": roof}


def mixed_split_report(steps: int, warmup: int) -> dict:
    """The chunked-prefill step mixed with decode rows (64 one-token rows over
    U{512..4096} + 8 x 512-token chunks over U{512..8192}-token prefixes),
    served three ways: one pa_prefill call over the whole varlen batch; the
    decode rows through pa_decode and the chunks through pa_prefill, back to
    back on one stream; and the same two calls on two streams at once (the
    decode on a second stream joined with events).  Medians of HIP-event times
    on the first stream, after a sustained warm-up."""
    c = wl.chunked_prefill_mixed()
    dev = place(c)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    nd = int((c.q_lens == 1).sum())
    assert np.all(c.q_lens[:nd] == 1) and np.all(c.q_lens[nd:] > 1)
    out = torch.empty((c.total_q_rows, c.num_q_heads, c.head_dim), dtype=torch.bfloat16, device="cuda")
    ws_all = pa.alloc_prefill_workspace(c.batch, c.total_q_rows, c.max_q_len, c.num_q_heads,
                                        c.num_kv_heads, c.max_blocks_per_seq)
    q_dec, out_dec = dev.q[:nd], out[:nd]
    tab_dec, len_dec = dev.block_table[:nd], dev.context_lens[:nd]
    ws_dec = pa.alloc_decode_workspace(nd, c.num_q_heads, c.num_kv_heads)
    q_chk, out_chk = dev.q[nd:], out[nd:]
    tab_chk, len_chk = dev.block_table[nd:].contiguous(), dev.context_lens[nd:].contiguous()
    cu_chk = (dev.cu_q[nd:] - nd).contiguous()
    max_dec = int(c.context_lens[:nd].max())
    rows_chk = c.total_q_rows - nd
    ws_chk = pa.alloc_prefill_workspace(c.batch - nd, rows_chk, c.max_q_len, c.num_q_heads,
                                        c.num_kv_heads, c.max_blocks_per_seq)
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    ev_fork, ev_join = torch.cuda.Event(), torch.cuda.Event()

    def one_call():
        pa.prefill(out, dev.q, dev.cu_q, dev.context_lens, c.max_q_len, dev.k_cache, dev.v_cache,
                   dev.block_table, c.scale, ws_all)

    def decode_rows(stream=None):
        pa.decode(out_dec, q_dec, dev.k_cache, dev.v_cache, tab_dec, len_dec, max_dec, c.scale, ws_dec,
                  stream=stream)

    def chunks():
        pa.prefill(out_chk, q_chk, cu_chk, len_chk, c.max_q_len, dev.k_cache, dev.v_cache, tab_chk,
                   c.scale, ws_chk)

    def two_calls():
        decode_rows()
        chunks()

    def two_streams():
        ev_fork.record(s0)
        s1.wait_event(ev_fork)
        decode_rows(stream=s1)
        chunks()
        ev_join.record(s1)
        s0.wait_event(ev_join)

    def two_streams_prefill_first():
        # the chunks' workgroups take the CUs first; the decode's fill the
        # CUs their shorter blocks leave idle towards the end
        ev_fork.record(s0)
        chunks()
        s1.wait_event(ev_fork)
        decode_rows(stream=s1)
        ev_join.record(s1)
        s0.wait_event(ev_join)

    res = {"workload": c.name, "decode_rows": nd, "chunk_rows": rows_chk}
    for label, fn in (("one_pa_prefill_call", one_call), ("decode_then_prefill_one_stream", two_calls),
                      ("decode_and_prefill_two_streams", two_streams),
                      ("prefill_then_decode_two_streams", two_streams_prefill_first)):
        _warm(fn, warmup)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record(s0)
            fn()
            e1.record(s0)
        torch.cuda.synchronize()
        res[label + "_ms"] = round(float(np.median([a.elapsed_time(b) for a, b in evs])), 4)
    fl = prefill_flops(c)
    best = min(res["decode_then_prefill_one_stream_ms"], res["decode_and_prefill_two_streams_ms"],
               res["prefill_then_decode_two_streams_ms"])
    res["causal_gflop"] = round(fl / 1e9, 3)
    res["best_TFLOPs"] = round(fl / (best * 1e-3) / 1e12, 1)
    del dev, out
    torch.cuda.empty_cache()
    return res


def decode_multi_report(name: str, steps: int, warmup: int) -> dict:
    """pa_decode_multi on a multi-query decode workload (several new tokens
    per sequence scored in one pass: the vector-ALU kernel up to 4 rows per
    (sequence, kv head), the matrix-core kernels for 5 to 16 and 17 to 32):
    the algorithmic
    bytes (every context's K/V rows once, q in, out written, table entries,
    lengths) over the HBM peak, HIP events around back-to-back launches."""
    c = wl.CONFIGS[name]()
    ql = int(c.q_lens[0])
    dev = place(c)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    out = torch.empty((c.total_q_rows, c.num_q_heads, c.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = pa.alloc_decode_multi_workspace(c.batch, ql, c.num_q_heads, c.num_kv_heads)

    def call():
        pa.decode_multi(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens, ql,
                        c.max_context_len, c.scale, ws)

    _warm(call, warmup)
    ms = _events_batch_ms(call, steps)
    kvb = int(c.context_lens.sum()) * c.num_kv_heads * c.head_dim * 2 * 2
    blocks = sum(wl.blocks_for(int(n)) for n in c.context_lens)
    alg = kvb + 2 * c.total_q_rows * c.num_q_heads * c.head_dim * 2 + 4 * blocks + 4 * c.batch
    gbs = alg / (ms * 1e-3) / 1e9
    rows = ql * c.num_q_heads // c.num_kv_heads
    kernel = ("decode_mfma_kernel" if rows > 16 else
              "decode_mfma16_kernel" if rows > 4 else "decode_split_kernel (several rows)")
    del dev, out, ws
    torch.cuda.empty_cache()
    return {"workload": c.name, "entry_point": "pa_decode_multi", "q_per_seq": ql,
            "rows_per_kv_head": rows, "decode_ms": round(ms, 4), "kv_GBps": round(kvb / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "algorithmic_bytes_per_launch": alg}}


def blocks_report(steps: int, warmup: int) -> dict:
    """pa_copy_blocks over 512 block pairs of a 2,048-block pool (8 kv heads:
    1 MiB of K+V per block, so 512 MiB read + 512 MiB written per call), and
    pa_swap_blocks of 256 blocks to a pinned host pool and back."""
    nb, hkv, n = 2048, 8, 512
    k, v = pa.alloc_cache(nb, hkv, "cuda", fill_bits=0x3F80)
    rng = np.random.default_rng(8)
    perm = rng.permutation(nb).astype(np.int32)
    pairs = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], axis=1).copy()).cuda()
    block_bytes = 2 * hkv * 256 * 128 * 2  # K and V of one block
    for _ in range(warmup):
        pa.copy_blocks(k, v, pairs)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        pa.copy_blocks(k, v, pairs)
        e1.record()
    torch.cuda.synchronize()
    cms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    cbytes = 2 * n * block_bytes
    m = 256
    hk = torch.empty((m,) + tuple(k.shape[1:]), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty((m,) + tuple(v.shape[1:]), dtype=torch.bfloat16, pin_memory=True)
    out_pairs = np.stack([perm[:m], np.arange(m, dtype=np.int32)], axis=1)
    in_pairs = out_pairs[:, ::-1].copy()
    times = {"out": [], "in": []}
    for i in range(warmup + steps):
        for kind, (sk, sv, dk, dv, pp) in (("out", (k, v, hk, hv, out_pairs)),
                                            ("in", (hk, hv, k, v, in_pairs))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pa.swap_blocks(sk, sv, dk, dv, pp)
            e1.record()
            torch.cuda.synchronize()
            if i >= warmup:
                times[kind].append(e0.elapsed_time(e1))
    sbytes = m * block_bytes
    res = {"copy_blocks_pairs": n, "copy_blocks_ms": round(cms, 4),
           "copy_blocks_GBps": round(cbytes / (cms * 1e-3) / 1e9, 1),
           "copy_blocks_frac_of_hbm_peak": round(cbytes / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    for kind in ("out", "in"):
        t = float(np.median(times[kind]))
        res[f"swap_{kind}_blocks"] = m
        res[f"swap_{kind}_ms"] = round(t, 4)
        res[f"swap_{kind}_GBps"] = round(sbytes / (t * 1e-3) / 1e9, 1)
    del k, v, hk, hv
    torch.cuda.empty_cache()
    return res


def block_manager_report(steps: int = 512) -> dict:
    """Host cost of the block manager in a decode loop: the batch of the
    256-sequence decode workload (its context lengths as prompts, every
    other sequence forked from its neighbour so that copy-on-write happens),
    then `steps` decode steps, each one pa_bm_append_batch for the whole
    batch plus the step's block table (pa_bm_block_table).  Also the same
    appends made one pa_bm_append call per sequence, for comparison."""
    case = wl.CONFIGS["qwen3_4b_decode"]()
    lens = [int(x) for x in case.context_lens]
    res = {"batch": len(lens), "steps": steps}
    for mode in ("batched", "per_sequence"):
        need = sum(-(-(n + steps) // 256) for n in lens) + len(lens)
        bm = pa.BlockManager(need)
        for i, n in enumerate(lens):
            if i % 2 == 1:
                bm.fork(i - 1, i)
            else:
                bm.allocate(i, n)
        seqs = list(range(len(lens)))
        width = -(-(max(lens) + steps) // 256)
        copies = 0
        t0 = time.perf_counter()
        for _ in range(steps):
            if mode == "batched":
                _, pairs = bm.append_batch(seqs)
                copies += len(pairs)
            else:
                for q in seqs:
                    copies += bm.append(q)[1] is not None
            bm.block_table(seqs, width)
        dt = time.perf_counter() - t0
        res[f"{mode}_us_per_step"] = round(dt / steps * 1e6, 2)
        res[f"{mode}_appends_per_s"] = round(steps * len(lens) / dt, 1)
        res[f"{mode}_copy_pairs"] = copies
    return res


# ---------------------------------------------------------------------------
# Profile summaries (rocprofv3 CSV -> short text/JSON under profiles/)

PROFILES = os.path.join(ROOT, "profiles")
# each kernel's source and the headers it includes; the digests below add the
# hipcc options it is compiled with
_CSRC = os.path.join(ROOT, "paged_kv_cache_237_amd", "csrc")
DECODE_SRC = tuple(os.path.join(_CSRC, f) for f in (
    "decode.hip", "decode_common.hpp", "pa_device.hpp", "pa_internal.hpp", "pa_common.hpp"))


def kernel_digest(paths, source_name: str) -> str:
    """Digest of what a kernel's code depends on: its source, the headers it
    includes and the hipcc options of its translation unit."""
    import hashlib
    from paged_kv_cache_237_amd import build as b
    flags = json.dumps([b.HIPCC_FLAGS, b.SOURCE_FLAGS.get(source_name, [])]).encode()
    return hashlib.sha256(source_digest(*paths).encode() + flags).hexdigest()[:16]


def source_digest(*paths: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def _read_csv(path: str):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_stats(stats_csv: str, out_md: str, command: str) -> None:
    """Kernel-trace statistics of a rocprofv3 run, as a short Markdown table."""
    rows = _read_csv(stats_csv)
    lines = ["# rocprofv3 kernel statistics", "", "Command (run from the repository root):", "",
             "```", command, "```", "",
             "Library kernels, the benchmark's load-only read-ceiling kernel and device copies "
             "only; the other kernels of the run are torch kernels that generate the seeded "
             "inputs before timing.", "",
             "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        if ("pa::" not in r["Name"] and "copyBuffer" not in r["Name"]
                and "stream_read_kernel" not in r["Name"]):
            continue
        name = r["Name"]
        short = name if len(name) < 70 else name[:67] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _pmc_per_kernel(counter_csv: str, counter: str):
    """Values of `counter` per dispatch, per kernel name."""
    acc = {}
    for r in _read_csv(counter_csv):
        if r.get("Counter_Name") != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def summarize_traffic(fetch_csv: str, write_csv: str, copy_mib: int, kernel_key: str,
                      out_json: str, commands, source=DECODE_SRC) -> dict:
    """HBM bytes per launch of the kernel whose name contains kernel_key, from
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the value the
    same counter reads for a plain device copy of copy_mib MiB."""
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")

    def pick(d, key):
        """Average over the dispatches of the kernel matching key."""
        hits = [(k, v) for k, v in d.items() if key in k]
        if not hits:
            raise SystemExit(f"no dispatch of a kernel matching {key!r}: {sorted(d)}")
        k, v = max(hits, key=lambda kv: len(kv[1]))
        return k, (sum(v) / len(v), len(v))

    def pick_copy(d):
        """The largest dispatch of the runtime's device copy: the copy of
        known size (torch's elementwise kernels are not candidates: the ones
        that fill the input pools write more than the probe copy)."""
        best = None
        for k, v in d.items():
            if "copyBuffer" in k:
                m = max(v)
                if best is None or m > best[1][0]:
                    best = (k, (m, 1))
        if best is None:
            raise SystemExit("no device copy dispatch in the counter CSV")
        return best

    known = copy_mib * 2**20
    kf, (kfv, kfn) = pick(fetch, kernel_key)
    kw, (kwv, kwn) = pick(write, kernel_key)
    cf, (cfv, _) = pick_copy(fetch)
    cw, (cwv, _) = pick_copy(write)
    f_scale = known / (cfv * 1024.0)
    w_scale = known / (cwv * 1024.0)
    res = {
        "kernel": kf, "dispatches": int(kfn),
        "fetch_kib_raw": kfv, "write_kib_raw": kwv,
        "copy_kernel": cf, "copy_bytes": known,
        "copy_fetch_kib_raw": cfv, "copy_write_kib_raw": cwv,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "fetch_bytes": kfv * 1024.0 * f_scale, "write_bytes": kwv * 1024.0 * w_scale,
        "traffic_bytes": kfv * 1024.0 * f_scale + kwv * 1024.0 * w_scale,
        "commands": list(commands),
    }
    if source == DECODE_SRC:
        res["decode_source_sha256_16"] = kernel_digest(DECODE_SRC, "decode.hip")
    else:
        res["source"] = os.path.relpath(source[0], ROOT)
        res["source_sha256_16"] = kernel_digest(source, os.path.basename(source[0]))
    json.dump(res, open(out_json, "w"), indent=1)
    return res


# the prefill kernel and the headers it includes; its compiler options are
# added to the digest from the build script's option lists (prefill_digest)
PREFILL_SRC = tuple(os.path.join(ROOT, "paged_kv_cache_237_amd", "csrc", f)
                    for f in ("prefill.hip", "pa_device.hpp", "pa_common.hpp", "pa_prefill.hpp"))
PREFILL_COUNTERS = os.path.join(PROFILES, "prefill_8x2048_sq_counters.json")


def prefill_digest() -> str:
    """Digest of what the prefill kernel's code depends on."""
    return kernel_digest(PREFILL_SRC, "prefill.hip")


def summarize_counters(out_md: str, kernel_key: str, csvs, commands) -> dict:
    """SQ / GRBM counters of the kernel whose name contains kernel_key,
    averaged over its dispatches (each value summed over the hardware
    instances), from one or more rocprofv3 --pmc counter CSVs; writes a
    Markdown table next to a JSON copy and returns the figures.  MFMA busy
    fraction = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE per XCD),
    with GRBM_GUI_ACTIVE taken from the same pass."""
    per_pass = []
    for path in csvs:
        vals = {}
        for r in _read_csv(path):
            if kernel_key not in r.get("Kernel_Name", ""):
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if not vals:
            raise SystemExit(f"no dispatch of a kernel matching {kernel_key!r} in {path}")
        per_pass.append({k: (sum(v) / len(v), len(v)) for k, v in vals.items()})
    merged = {}
    for d in per_pass:
        for k, (v, n) in d.items():
            merged.setdefault(k, (v, n))
    simds = 256 * 4
    xcds = 8
    ratios = {}
    for d in per_pass:
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d:
            busy = d["SQ_VALU_MFMA_BUSY_CYCLES"][0]
            ratios["mfma_busy_frac"] = busy / (simds * d["GRBM_GUI_ACTIVE"][0] / xcds)
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in d:
                ratios["valu_coexec_frac_of_mfma_busy"] = d["SQ_VALU_MFMA_COEXEC_CYCLES"][0] / busy
        if "SQ_WAIT_INST_ANY" in d and "SQ_WAVE_CYCLES" in d:
            ratios["wait_inst_any_frac_of_wave_cycles"] = d["SQ_WAIT_INST_ANY"][0] / d["SQ_WAVE_CYCLES"][0]
        if "SQ_WAIT_INST_LDS" in d and "SQ_WAVE_CYCLES" in d:
            ratios["wait_inst_lds_frac_of_wave_cycles"] = d["SQ_WAIT_INST_LDS"][0] / d["SQ_WAVE_CYCLES"][0]
    res = {"kernel_key": kernel_key, "counters": {k: v for k, (v, _) in sorted(merged.items())},
           "dispatches": min(n for _, n in merged.values()), "ratios": ratios,
           "prefill_source_sha256_16": prefill_digest(), "commands": list(commands)}
    lines = [f"# `{kernel_key}` SQ counters", "",
             "Commands (run from the repository root, one pass each; values are summed over the "
             "hardware instances and averaged over the kernel's dispatches):", "", "```",
             *commands, "```", "", "| counter | per dispatch |", "|---|---|"]
    lines += [f"| {k} | {v:.4g} |" for k, v in res["counters"].items()]
    lines += ["", "| ratio | value |", "|---|---|"]
    lines += [f"| {k} | {v:.3f} |" for k, v in ratios.items()]
    open(out_md, "w").write("\n".join(lines) + "\n")
    json.dump(res, open(os.path.splitext(out_md)[0] + ".json", "w"), indent=1)
    return res


def recorded_prefill_counters():
    """MFMA busy fraction of the prefill kernel from the committed counter
    summary, if the prefill source has not changed since it was taken."""
    if not os.path.exists(PREFILL_COUNTERS):
        return None
    rec = json.load(open(PREFILL_COUNTERS))
    if rec.get("prefill_source_sha256_16") != prefill_digest():
        return None
    return rec.get("ratios")


STORE_SRC = tuple(os.path.join(_CSRC, f) for f in (
    "store_kv.hip", "pa_device.hpp", "pa_internal.hpp", "pa_common.hpp"))
STORE_TRAFFIC = os.path.join(PROFILES, "store_16384_tokens_traffic.json")


def recorded_store_traffic():
    """HBM bytes per launch of the 16,384-token store from the committed
    counter summary, if the store kernel source has not changed since."""
    if not os.path.exists(STORE_TRAFFIC):
        return None
    rec = json.load(open(STORE_TRAFFIC))
    if rec.get("source_sha256_16") != kernel_digest(STORE_SRC, "store_kv.hip"):
        return None
    return int(round(rec["traffic_bytes"]))


PREFILL_TRAFFIC = os.path.join(PROFILES, "prefill_8x2048_traffic.json")


def recorded_prefill_traffic():
    """HBM bytes per launch of the 8 x 2048 prefill from the committed
    counter summary, if the prefill sources have not changed since."""
    if not os.path.exists(PREFILL_TRAFFIC):
        return None
    rec = json.load(open(PREFILL_TRAFFIC))
    if rec.get("source_sha256_16") != prefill_digest():
        return None
    return int(round(rec["traffic_bytes"]))


def recorded_traffic(workload: str):
    """Traffic per launch from the committed counter summary of this workload,
    if the decode kernel source has not changed since it was taken."""
    path = os.path.join(PROFILES, f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("decode_source_sha256_16") != kernel_digest(DECODE_SRC, "decode.hip"):
        return None
    return int(round(rec["traffic_bytes"]))


def _oracle_threads() -> int:
    from threadpoolctl import threadpool_info
    return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))


def cpu_baseline(case: wl.PagedCase, budget_s: float = 10.0, max_seqs: int = 0) -> dict:
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload: whole sequences in batch order until about budget_s of
    oracle time; with max_seqs > 0 only the first max_seqs sequences are built
    and the sample cycles over them (a 131,072-token sequence takes ~3 s of
    oracle time but ~12 s to build its host pools, which are not timed)."""
    import oracle

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from paged_harness import oracle_pools  # noqa: E402

    q = wl.bits_to_numpy(case.q_all())
    pools = {}
    done_ctx, done_seqs, spent = 0, 0, 0.0
    cycle = case.batch if max_seqs <= 0 else min(max_seqs, case.batch)
    while spent < budget_s:
        b = done_seqs % cycle
        if b not in pools:
            pools[b] = oracle_pools(case, [b], poison=False)
        kp, vp = pools[b]
        t0 = time.perf_counter()
        oracle.decode_seq(q[b], kp, vp, case.block_table[b], int(case.context_lens[b]), case.scale)
        spent += time.perf_counter() - t0
        done_ctx += int(case.context_lens[b])
        done_seqs += 1
        if len(pools) > 8:
            pools.pop(next(iter(pools)))
    del pools
    bytes_done = done_ctx * case.num_kv_heads * case.head_dim * 2 * 2
    which = "in batch order" if cycle == case.batch else f"cycling over the first {cycle}"
    return {"value": round(bytes_done / spent / 1e9, 4), "unit": "GB/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"{case.name}: float64 oracle decode of {done_seqs} whole sequences {which} "
                      f"({done_ctx} attended tokens x {case.num_q_heads} q heads, "
                      f"{spent:.1f} s of oracle time; {done_ctx / spent:.0f} attended tokens/s); "
                      f"GB/s counts the same algorithmic K/V bytes as the GPU figure"}


def cpu_baseline_prefill(case: wl.PagedCase, budget_s: float = 10.0) -> dict:
    """The oracle's causal prefill timed on the host cores: whole sequences in
    batch order until about budget_s of oracle time, reported in causal
    TFLOP/s (the same FLOP count as the GPU figure)."""
    import oracle

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from paged_harness import oracle_pools  # noqa: E402

    q = wl.bits_to_numpy(case.q_all())
    flops, seqs, spent = 0, 0, 0.0
    pools = None
    while spent < budget_s and seqs < 4 * case.batch:
        b = seqs % case.batch
        if pools is None:
            pools = oracle_pools(case, poison=False)
        kp, vp = pools
        lo, hi = int(case.q_offsets[b]), int(case.q_offsets[b + 1])
        t0 = time.perf_counter()
        oracle.prefill_seq(q[lo:hi], kp, vp, case.block_table[b], int(case.context_lens[b]), case.scale)
        spent += time.perf_counter() - t0
        ql, n = hi - lo, int(case.context_lens[b])
        flops += 4 * case.head_dim * case.num_q_heads * (ql * (n - ql + 1) + ql * (ql - 1) // 2)
        seqs += 1
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"{case.name}: float64 oracle causal prefill of {seqs} whole sequences in batch "
                      f"order ({flops / 1e9:.1f} causal GFLOP, {spent:.1f} s of oracle time)"}


def versions() -> dict:
    """Software and device the figures were measured with."""
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    p = torch.cuda.get_device_properties(0)
    return {"torch": torch.__version__, "torch_hip": torch.version.hip, "rocm": rocm,
            "device": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "python": sys.version.split()[0]}


def decode_split_plan(case: wl.PagedCase, cus: int, append: bool = True) -> dict:
    """How a decode launch of this workload cuts its work (the rule the
    library applies on the host and in the kernel's prologue): every
    (sequence, kv head) is a segment of ceil(n / 64) tiles of 64 tokens (n =
    the context, minus the appended token for pa_decode_append), the segments
    are laid end to end and cut into one run per wave, runs weighted 12 on
    even- and 11 on odd-numbered XCDs (equal runs when there are too few
    tiles); a segment whose first and last tiles fall in different runs is
    merged from partial states."""
    g = case.num_q_heads // case.num_kv_heads
    nw = 4 if g == 8 else 8
    cap = case.max_blocks_per_seq * case.block_size
    ctx = np.clip(case.context_lens.astype(np.int64), 0, cap)
    streamed = np.where(ctx > 0, ctx - 1, 0) if append else ctx
    nt = (streamed + 63) // 64
    hkv = case.num_kv_heads
    total = int(nt.sum()) * hkv
    tiles_upper = case.batch * hkv * ((case.max_context_len + 63) // 64)
    n_waves = max(1, min(cus * nw, tiles_upper))
    we, wo = 12, 11

    def weight_before(w):
        blk, wv = w // nw, w % nw
        s0 = (blk >> 1) * nw * (we + wo)
        return s0 + nw * we + wv * wo if blk & 1 else s0 + wv * we

    ssum = weight_before(n_waves)
    weighted = total * min(we, wo) >= ssum
    per = 0 if weighted else -(-total // n_waves)

    def run_start(w):
        if per:
            return min(w * per, total)
        return total if w >= n_waves else total * weight_before(w) // ssum

    starts = np.array([run_start(w) for w in range(n_waves + 1)], dtype=np.int64)
    seg_nt = np.repeat(nt, hkv)
    seg_lo = np.concatenate([[0], np.cumsum(seg_nt)[:-1]])
    live = seg_nt > 0
    w_first = np.searchsorted(starts, seg_lo[live], side="right") - 1
    w_last = np.searchsorted(starts, seg_lo[live] + seg_nt[live] - 1, side="right") - 1
    lens = np.diff(starts)
    return {"waves": int(n_waves), "workgroups": int(-(-n_waves // nw)), "waves_per_workgroup": nw,
            "total_tiles": total, "tile_tokens": 64,
            "runs": "weighted 12:11 (even:odd XCD)" if weighted else f"equal, {per} tiles",
            "tiles_per_wave_min_max": [int(lens.min()), int(lens.max())],
            "segments": int(live.sum()), "segments_merged": int((w_first != w_last).sum())}


def decode_entry(case: wl.PagedCase, t: dict, cus: int, ceiling=None) -> dict:
    """Figures of one decode workload from time_decode's timings: the step
    rate, the step kernel's roofline (pa_decode_append: HIP events around
    single launches on the stream the kernel runs on), plain pa_decode's,
    and the split plan."""
    g = case.num_q_heads // case.num_kv_heads
    dbytes, abytes = decode_bytes(case), append_bytes(case)
    sbytes = store_bytes(int((case.context_lens > 0).sum()), case.num_kv_heads)
    sum_ctx = int(case.context_lens.sum())
    step_gbs = (dbytes + sbytes) / (t["step_ms"] * 1e-3) / 1e9
    app_gbs = abytes / (t["append_ms"] * 1e-3) / 1e9
    dec_gbs = dbytes / (t["decode_ms"] * 1e-3) / 1e9
    flushed = t["decode_ms_flushed"]
    e = {
        "workload": case.name,
        "step_ms": round(t["step_ms"], 4), "step_GBps": round(step_gbs, 1),
        "pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "attended_tokens_per_s": round(sum_ctx / (t["step_ms"] * 1e-3), 1),
        "sum_context_len": sum_ctx,
        "step_graph_replay_ms": round(t["step_graph_ms"], 4) if "step_graph_ms" in t else None,
        "two_call_step": {"ms": round(t["two_call_step_ms"], 4),
                          "GBps": round((dbytes + sbytes) / (t["two_call_step_ms"] * 1e-3) / 1e9, 1),
                          "graph_replay_ms": (round(t["two_call_step_graph_ms"], 4)
                                              if "two_call_step_graph_ms" in t else None),
                          "calls": "pa_store_kv + pa_decode"},
        "append_ms": round(t["append_ms"], 4),
        "decode_ms": round(t["decode_ms"], 4),
        "decode_ms_caches_flushed": {"median": round(float(np.median(flushed)), 4),
                                     "min": round(float(np.min(flushed)), 4),
                                     "max": round(float(np.max(flushed)), 4)},
        "store_ms": round(t["store_ms"], 4),
        "roofline": {"bound": "hbm",
                     "kernel": f"decode_split_kernel<{g}, false, true> (pa_decode_append: the step's "
                               "store and split-context decode with fused merge)",
                     "achieved": round(app_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(app_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(case.name),
                     "algorithmic_bytes_per_launch": abytes,
                     "launch_us": round(t["append_ms"] * 1e3, 2)},
        "pa_decode_roofline": {"bound": "hbm", "kernel": f"decode_split_kernel<{g}, false, false> (pa_decode)",
                               "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes_per_launch": dbytes},
        "split_plan": decode_split_plan(case, cus),
    }
    if ceiling is not None:
        # the step kernel against what a load-only launch of its shape and
        # size streams on this machine (non-temporal loads, as the kernel's)
        e["hbm_read_ceiling_measured"] = ceiling
        e["append_frac_of_same_size_ceiling"] = round(
            ceiling["step_bytes_nt"]["us"] / (t["append_ms"] * 1e3), 4)
    return e


DEFAULT_WORKLOAD = "long_context_decode"
DECODE_WORKLOADS = ("long_context_decode", "qwen3_4b_decode", "qwen3_0.6b_decode")


# workloads --extra-only can time alone: pa_prefill batches, pa_decode_multi
# batches, the block copies / swaps
EXTRA_ONLY = ("chunked_prefill_mixed", "multi_query_decode", "spec_verify_decode", "long_prefix_chunk",
              "long_chunk_with_decode", "multi_query_decode_multi", "spec_verify_decode_multi",
              "spec_verify_decode_g4_multi", "blocks")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(wl.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workload shapes")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timings of the step (the headline step is eager)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time store + prefill of the 8 x 2048 prompt batch (for profiling)")
    ap.add_argument("--extra-only", choices=EXTRA_ONLY, default=None,
                    help="only time this one extra workload (for a kernel trace of it alone): a "
                         "pa_prefill batch, a pa_decode_multi batch (suffix _multi) or the block copies")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "OUT_MD", "COMMAND"),
                    help="write a Markdown summary of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--summarize-traffic", nargs=5,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_MIB", "KERNEL_KEY", "OUT_JSON"),
                    help="write the per-launch HBM traffic of a kernel from FETCH_SIZE / "
                         "WRITE_SIZE counter CSVs and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="OUT_MD KERNEL_KEY CSV [CSV ...]: write a summary of SQ/GRBM counter "
                         "CSVs of one kernel (rocprofv3 --pmc passes) and exit")
    ap.add_argument("--traffic-source", choices=("decode", "store", "prefill"), default="decode",
                    help="kernel whose source digest a traffic summary records (default: decode)")
    ap.add_argument("--commands", nargs="*", default=[],
                    help="the profiler commands recorded in a traffic summary")
    args = ap.parse_args(argv)
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return 0
    if args.summarize_traffic:
        f, w, mib, key, out = args.summarize_traffic
        src = {"decode": DECODE_SRC, "store": STORE_SRC, "prefill": PREFILL_SRC}[args.traffic_source]
        print(json.dumps(summarize_traffic(f, w, int(mib), key, out, args.commands, src)))
        return 0
    if args.summarize_counters:
        out_md, key, *csvs = args.summarize_counters
        print(json.dumps(summarize_counters(out_md, key, csvs, args.commands)))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the path is single-GPU; sharding is described in the design notes)",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    pa.lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    if args.prefill_only:
        print(json.dumps({"prefill": prefill_report(args.steps, args.warmup)}), flush=True)
        copy_probe(args.copy_probe_mib)
        return 0
    if args.extra_only:
        name = args.extra_only
        if name == "blocks":
            res = blocks_report(args.steps, args.warmup)
        elif name.endswith("_multi"):
            res = decode_multi_report(name[:-len("_multi")], args.steps, args.warmup)
        else:
            res = varlen_report(name, args.steps, args.warmup)
        print(json.dumps({name: res}), flush=True)
        return 0

    case = wl.CONFIGS[args.workload]()
    if case.kind != "decode":
        print("the headline step is a decode step; choose a decode workload", file=sys.stderr)
        return 2
    print(f"[bench] {case.name}: B={case.batch} sum_ctx={int(case.context_lens.sum())}",
          file=sys.stderr, flush=True)
    t = time_decode(case, args.steps, args.warmup)
    copy_probe(args.copy_probe_mib)
    ceiling = read_ceiling([append_bytes(case), 4 << 30], ["step_bytes", "4GiB"])
    head = decode_entry(case, t, cus, ceiling)
    line = {
        "metric": METRIC,
        "value": head.pop("step_GBps"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("step_ms"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1) bf16 values, shuffled physical blocks)",
        "config": {"workload": case.name, "batch": case.batch, "num_q_heads": case.num_q_heads,
                   "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
                   "block_size": case.block_size, "sum_context_len": int(case.context_lens.sum()),
                   "max_context_len": case.max_context_len, "num_blocks": case.num_blocks,
                   "parallelism": "single GPU"},
        "roofline": head.pop("roofline"),
        "step_launch": "one pa_decode_append launch per step (store of the new tokens + decode), "
                       "launched back to back on one stream",
        "versions": versions(),
    }
    head.pop("workload")
    line.update(head)
    if not args.no_extra:
        extra = {}
        for name in DECODE_WORKLOADS:
            if name == case.name:
                continue
            c = wl.CONFIGS[name]()
            print(f"[bench] extra {name}", file=sys.stderr, flush=True)
            tc = time_decode(c, max(10, args.steps // 5), 3)
            cl = read_ceiling([append_bytes(c)], ["step_bytes"])
            extra[name] = decode_entry(c, tc, cus, cl)
        print("[bench] extra prefill_8x2048", file=sys.stderr, flush=True)
        extra["prefill_8x2048"] = prefill_report(max(30, args.steps // 5), 3)
        for name in ("chunked_prefill_mixed", "multi_query_decode", "spec_verify_decode",
                     "long_prefix_chunk", "long_chunk_with_decode"):
            print(f"[bench] extra {name}", file=sys.stderr, flush=True)
            extra[name] = varlen_report(name, max(30, args.steps // 5), 3)
        for name in ("multi_query_decode", "spec_verify_decode", "spec_verify_decode_g4"):
            print(f"[bench] extra {name} (pa_decode_multi)", file=sys.stderr, flush=True)
            extra[f"{name}_multi"] = decode_multi_report(name, max(20, args.steps // 5), 3)
        print("[bench] extra block copy / swap", file=sys.stderr, flush=True)
        extra["blocks"] = blocks_report(max(10, args.steps // 5), 3)
        print("[bench] extra block manager (host)", file=sys.stderr, flush=True)
        extra["block_manager"] = block_manager_report()
        line["extra"] = extra
    # last: what launches work on a second stream (see time_decode_graphs)
    if not args.no_graph:
        print("[bench] graph replays", file=sys.stderr, flush=True)
        entries = [(case, line)] + [(wl.CONFIGS[n](), line["extra"][n]) for n in DECODE_WORKLOADS
                                    if not args.no_extra and n in line["extra"]]
        for c, e in entries:
            tg = time_decode_graphs(c, args.steps if c is case else max(10, args.steps // 5),
                                    args.warmup if c is case else 3)
            e["step_graph_replay_ms"] = round(tg["step_graph_ms"], 4)
            e["two_call_step"]["graph_replay_ms"] = round(tg["two_call_step_graph_ms"], 4)
    if not args.no_extra:
        print("[bench] extra chunked_prefill_mixed split by kernel", file=sys.stderr, flush=True)
        line["extra"]["chunked_prefill_mixed_split"] = mixed_split_report(max(30, args.steps // 5), 3)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(case, max_seqs=2 if case.max_context_len > 65536 else 0)
        if not args.no_extra:
            for name in ("qwen3_0.6b_decode",):
                if name in line["extra"]:
                    print(f"[bench] cpu baseline (oracle) {name}", file=sys.stderr, flush=True)
                    line["extra"][name]["cpu_baseline"] = cpu_baseline(wl.CONFIGS[name]())
            print("[bench] cpu baseline (oracle) prefill_8x2048", file=sys.stderr, flush=True)
            line["extra"]["prefill_8x2048"]["cpu_baseline"] = cpu_baseline_prefill(wl.prefill_8x2048())
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
