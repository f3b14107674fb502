"""One fixed decode input under different split-context plans: the number of
runs the work list is cut into is fixed with the library's testing aid
(pa_set_decode_waves) -- 1 (every context streamed whole by one wave), 2, 7,
the automatic count, 64, and the most the workspace allows (one 64-token
tile per run here, so every context longer than one tile is merged from
partial states).  Every plan must meet the oracle bar, for pa_decode and for
pa_decode_append (whose merges also fold in the appended token), and for a
fixed plan the result must not depend on where the blocks sit in the pool
(same logical contents under another block permutation: identical bits)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_237_amd as pa
import workloads as wl
from device_case import new_rows
from paged_harness import bf16_out_to_f64, compare, oracle_pools, place

pytestmark = pytest.mark.gpu

LENS = [1, 63, 64, 65, 700, 3000, 4096, 257]
PLANS = [1, 2, 7, 0, 64, 1 << 20]  # 0 = automatic; the last is clamped to 8 per CU


def _cases(hq):
    a = wl.make_case(f"plans_{hq}", "decode", 120 + hq, LENS, hq, 8, num_blocks=60)
    b = wl.make_case(f"plans_{hq}", "decode", 120 + hq, LENS, hq, 8, num_blocks=60,
                     rng=np.random.default_rng(4242))
    assert not np.array_equal(a.block_table, b.block_table)
    return a, b


def _decode(dev, append):
    c = dev.case
    out = torch.full((c.batch, c.num_q_heads, c.head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    ws = pa.alloc_decode_workspace(c.batch, c.num_q_heads, c.num_kv_heads)
    if append:
        k_new, v_new = new_rows(dev)
        pa.decode_append(out, dev.q, k_new, v_new, dev.k_cache, dev.v_cache, dev.block_table,
                         dev.context_lens, c.max_context_len, c.scale, ws)
    else:
        pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
        pa.decode(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens,
                  c.max_context_len, c.scale, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("hq", [16, 32, 64])
@pytest.mark.parametrize("append", [False, True])
def test_split_plans_agree_with_oracle_and_ignore_placement(hq, append):
    ca, cb = _cases(hq)
    kp, vp = oracle_pools(ca)
    ref = oracle.decode(wl.bits_to_numpy(ca.q_all()), kp, vp, ca.block_table, ca.context_lens,
                        ca.scale)
    outs = {}
    try:
        for waves in PLANS:
            print(f"[plans] hq={hq} append={append} waves={waves}", flush=True)
            pa.set_decode_waves(waves)
            oa = _decode(place(ca), append)
            ob = _decode(place(cb), append)
            assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), \
                f"waves={waves}: placement changed the bits"
            compare(bf16_out_to_f64(oa), ref, f"plans hq={hq} waves={waves} append={append}")
            outs[waves] = oa.view(torch.int16).clone()
    finally:
        pa.set_decode_waves(0)
    # one wave per context and the automatic plan really are different cuts:
    # their results differ somewhere by rounding (else the knob did nothing)
    assert not torch.equal(outs[1], outs[1 << 20])


@pytest.mark.parametrize("hq,ql", [(16, 6), (32, 5)])
def test_multi_row_split_plans(hq, ql):
    """pa_decode_multi with 12 or 20 rows per (sequence, kv head) -- the
    matrix-core kernels, whose partial records hold 16 and 32 rows -- under
    the same plans, against the oracle's causal attention."""
    case = wl.make_case(f"plans_multi_{hq}", "prefill", 140 + hq, [ql, 63 + ql, 700, 3000, 4096, 257],
                        hq, 8, q_lens=[ql] * 6, num_blocks=40)
    dev = place(case)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    kp, vp = oracle_pools(case)
    q = wl.bits_to_numpy(case.q_all())
    ref = np.concatenate([oracle.prefill_seq(q[b * ql:(b + 1) * ql], kp, vp, case.block_table[b],
                                             int(case.context_lens[b]), case.scale)
                          for b in range(case.batch)])
    ws = pa.alloc_decode_multi_workspace(case.batch, ql, hq, 8)
    outs = {}
    try:
        for waves in PLANS:
            print(f"[plans multi] hq={hq} ql={ql} waves={waves}", flush=True)
            pa.set_decode_waves(waves)
            out = torch.full((case.batch * ql, hq, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
            pa.decode_multi(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens, ql,
                            case.max_context_len, case.scale, ws)
            torch.cuda.synchronize()
            compare(bf16_out_to_f64(out), ref, f"plans multi hq={hq} waves={waves}")
            outs[waves] = out.view(torch.int16).clone()
    finally:
        pa.set_decode_waves(0)
    assert not torch.equal(outs[1], outs[1 << 20])
