"""Benchmark of the paged KV-cache hot path on one MI355X.

One step = the whole path over one batch: pa_store_kv of each sequence's new
token, then pa_decode over every sequence's full paged context.  The default
workload is the Qwen3-0.6B-shaped decode layer (batch 64, context lengths
uniform on 512..4096, 16 query / 8 kv heads, head dim 128, 256-token blocks,
physical blocks shuffled, pool +10 %).  Inputs are seeded synthetic data
placed in HBM before timing.  Other workloads are reported under "extra"
(they are parity-test shapes; the headline line is the one above).

Prints ONE JSON line.  `--gpus N` with N > 1 exits: this build runs on one
GPU only.
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


def place(case):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from paged_harness import place as _place  # noqa: E402
    return _place(case)


def time_decode(case: wl.PagedCase, steps: int, warmup: int):
    """Times `steps` decode steps (store + decode) after `warmup`; returns
    (ms_per_step, decode_ms_avg, store_ms_avg)."""
    dev = place(case)
    out = torch.empty((case.batch, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    ws = pa.alloc_decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
        if ev is not None:
            ev[1].record(stream)
        pa.decode(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens,
                  case.max_context_len, case.scale, ws)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    sto = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    del dev
    torch.cuda.empty_cache()
    return wall * 1e3 / steps, dec, sto


def prefill_flops(case: wl.PagedCase) -> int:
    """Causal FLOPs of one pa_prefill: 4*D per (query row, visible key) pair
    per query head (q.k and p.v, a multiply and an add each)."""
    pairs = 0
    for b in range(case.batch):
        ql, n = int(case.q_lens[b]), int(case.context_lens[b])
        first = n - ql + 1  # keys seen by the first query row
        pairs += ql * first + ql * (ql - 1) // 2
    return 4 * case.head_dim * case.num_q_heads * pairs


def time_prefill(case: wl.PagedCase, steps: int, warmup: int):
    """Times store (all prompt tokens) + prefill; returns (store_ms, prefill_ms)."""
    dev = place(case)
    out = torch.empty((case.total_q_rows, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
        if ev is not None:
            ev[1].record(stream)
        pa.prefill(out, dev.q, dev.cu_q, dev.context_lens, case.max_q_len, dev.k_cache,
                   dev.v_cache, dev.block_table, case.scale)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    sto = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    pre = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    del dev
    torch.cuda.empty_cache()
    return sto, pre


def prefill_report(steps: int, warmup: int) -> dict:
    c = wl.prefill_8x2048()
    sto, pre = time_prefill(c, steps, warmup)
    fl = prefill_flops(c)
    sb = store_bytes(c.total_kv_rows, c.num_kv_heads)
    tf = fl / (pre * 1e-3) / 1e12
    return {"workload": c.name, "prefill_ms": round(pre, 4), "causal_gflop": round(fl / 1e9, 3),
            "prefill_TFLOPs": round(tf, 1), "frac_of_bf16_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
            "store_ms": round(sto, 4), "store_tokens": c.total_kv_rows,
            "store_GBps": round(sb / (sto * 1e-3) / 1e9, 1),
            "store_frac_of_hbm_peak": round(sb / (sto * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def cpu_baseline(case: wl.PagedCase, budget_s: float = 10.0) -> dict:
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload: whole sequences in batch order (wrapping around to the
    first sequence again) until about budget_s of oracle time."""
    import oracle
    from threadpoolctl import threadpool_info

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from paged_harness import oracle_pools  # noqa: E402

    q = wl.bits_to_numpy(case.q_all())
    pools = {}
    done_ctx, done_seqs, spent = 0, 0, 0.0
    while spent < budget_s:
        b = done_seqs % case.batch
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
    bytes_done = done_ctx * case.num_kv_heads * case.head_dim * 2 * 2
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(bytes_done / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{case.name}: float64 oracle decode of {done_seqs} whole sequences in "
                      f"batch order ({done_ctx} attended tokens x {case.num_q_heads} q heads, "
                      f"{spent:.1f} s of oracle time; {done_ctx / spent:.0f} attended tokens/s); "
                      f"GB/s counts the same algorithmic K/V bytes as the GPU figure"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_0.6b_decode", choices=sorted(wl.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workload shapes")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time store + prefill of the 8 x 2048 prompt batch (for profiling)")
    args = ap.parse_args(argv)
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

    if args.prefill_only:
        print(json.dumps({"prefill": prefill_report(args.steps, args.warmup)}), flush=True)
        return 0

    case = wl.CONFIGS[args.workload]()
    if case.kind != "decode":
        print("the headline step is a decode step; choose a decode workload", file=sys.stderr)
        return 2
    print(f"[bench] {case.name}: B={case.batch} sum_ctx={int(case.context_lens.sum())}",
          file=sys.stderr, flush=True)
    ms_step, dec_ms, sto_ms = time_decode(case, args.steps, args.warmup)
    dbytes = decode_bytes(case)
    sbytes = store_bytes(case.batch, case.num_kv_heads)
    sum_ctx = int(case.context_lens.sum())
    step_gbs = (dbytes + sbytes) / (ms_step * 1e-3) / 1e9
    dec_gbs = dbytes / (dec_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1) bf16 values, shuffled physical blocks)",
        "config": {"workload": case.name, "batch": case.batch, "num_q_heads": case.num_q_heads,
                   "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
                   "block_size": case.block_size, "sum_context_len": sum_ctx,
                   "max_context_len": case.max_context_len, "num_blocks": case.num_blocks,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "attended_tokens_per_s": round(sum_ctx / (ms_step * 1e-3), 1),
        "decode_ms": round(dec_ms, 4),
        "store_ms": round(sto_ms, 4),
        "roofline": {"bound": "hbm", "kernel": "pa_decode (split-context pass + merge pass)",
                     "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": dbytes},
    }
    if not args.no_extra:
        extra = {}
        for name in ("qwen3_4b_decode", "long_context_decode"):
            c = wl.CONFIGS[name]()
            print(f"[bench] extra {name}", file=sys.stderr, flush=True)
            m, d, s = time_decode(c, max(10, args.steps // 5), 3)
            b = decode_bytes(c)
            extra[name] = {"decode_ms": round(d, 4), "decode_GBps": round(b / (d * 1e-3) / 1e9, 1),
                           "frac_of_hbm_peak": round(b / (d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "attended_tokens_per_s": round(int(c.context_lens.sum()) / (d * 1e-3), 1),
                           "sum_context_len": int(c.context_lens.sum())}
        print("[bench] extra prefill_8x2048", file=sys.stderr, flush=True)
        extra["prefill_8x2048"] = prefill_report(max(10, args.steps // 5), 3)
        line["extra"] = extra
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
