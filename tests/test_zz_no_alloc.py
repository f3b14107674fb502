"""pa_decode_append_noalloc on the GPU: the allocation-free decode step
(library-owned scratch instead of a caller workspace) against
pa_decode_append with a workspace, through the C ABI.  Two calls in a row on
the one per-device scratch, the second with a smaller batch: outputs and the
caches' bytes must be identical to the workspace entry point's (same
kernel, same work plan), and a batch too large for the scratch is refused
before anything is launched."""

import numpy as np
import pytest
import torch

import paged_kv_cache_237_amd as pa
import workloads as wl
from device_case import new_rows
from paged_harness import bf16_out_to_f64, compare, oracle_pools, place

import oracle

pytestmark = pytest.mark.gpu


def _step(case, noalloc):
    """One decode step of `case` on fresh caches: returns (out, k_cache, v_cache)."""
    dev = place(case)
    k_new, v_new = new_rows(dev)
    out = torch.full((case.batch, case.num_q_heads, case.head_dim), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    if noalloc:
        pa.decode_append_noalloc(out, dev.q, k_new, v_new, dev.k_cache, dev.v_cache,
                                 dev.block_table, dev.context_lens, case.max_context_len, case.scale)
    else:
        ws = pa.alloc_decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads)
        pa.decode_append(out, dev.q, k_new, v_new, dev.k_cache, dev.v_cache, dev.block_table,
                         dev.context_lens, case.max_context_len, case.scale, ws)
    torch.cuda.synchronize()
    return out, dev


def _same(case):
    print(f"[noalloc] {case.name} B={case.batch} Hq={case.num_q_heads} Hkv={case.num_kv_heads}",
          flush=True)
    got, gdev = _step(case, True)
    ref, rdev = _step(case, False)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), case.name
    assert torch.equal(gdev.k_cache.view(torch.int16), rdev.k_cache.view(torch.int16))
    assert torch.equal(gdev.v_cache.view(torch.int16), rdev.v_cache.view(torch.int16))
    return got


def test_noalloc_matches_workspace_entry_point_twice_shrinking():
    """A Qwen3-4B-shaped step (256 sequences, many cut segments), then a
    smaller batch on the same scratch; the second call also shows the
    counters were left at zero by the first."""
    big = wl.qwen3_4b_decode()
    _same(big)
    small = wl.make_case("noalloc_small", "decode", 91, [1, 2, 63, 64, 65, 700, 3000, 9000], 16, 8)
    out = _same(small)
    # and against the oracle, to the usual bar
    kp, vp = oracle_pools(small)
    ref = oracle.decode(wl.bits_to_numpy(small.q_all()), kp, vp, small.block_table,
                        small.context_lens, small.scale)
    compare(bf16_out_to_f64(out), ref, "noalloc small")


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    """More sequences than the fixed scratch holds: PA_ERR_WORKSPACE, and the
    output is left untouched (nothing launched)."""
    b, hq, hkv = 4096, 32, 8
    assert pa.decode_workspace_size(b, hq, hkv) > pa.NOALLOC_SCRATCH_BYTES
    k, v = pa.alloc_cache(4, hkv, "cuda", fill_bits=0)
    q = torch.zeros((b, hq, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    kn = torch.zeros((b, hkv, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((b, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones(b, dtype=torch.int32, device="cuda")
    with pytest.raises(pa.PAError) as ei:
        pa.decode_append_noalloc(out, q, kn, kn, k, v, table, lens, 1, 0.1)
    assert ei.value.status == -5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
