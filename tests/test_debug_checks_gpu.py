"""The library's debug mode (pa_set_debug_checks / PA_DEBUG=1): a small
kernel checks the data-dependent preconditions of a call on the device before
the call's own kernels run.  Valid calls must pass and give the same bits as
without the checks; each violated precondition must come back as
PA_ERR_PRECONDITION with the outputs untouched (the call's kernels never
ran, so the poisoned buffers still hold their poison)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_237_amd as pa
import workloads as wl
from paged_harness import place

pytestmark = pytest.mark.gpu


@pytest.fixture
def checks_on():
    prev = pa.set_debug_checks(True)
    yield
    pa.set_debug_checks(prev)


def expect_precondition(fn, words):
    with pytest.raises(pa.PAError) as e:
        fn()
    assert e.value.status == -11, e.value
    for w in words:
        assert w in e.value.detail, e.value.detail


def test_valid_calls_pass_with_identical_results(checks_on):
    case = wl.qwen3_0_6b_decode()
    dev = place(case)
    ws = pa.alloc_decode_workspace(case.batch, 16, 8)
    outs = []
    for on in (True, False):
        pa.set_debug_checks(on)
        pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
        out = torch.empty((case.batch, 16, 128), dtype=torch.bfloat16, device="cuda")
        pa.decode(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens,
                  case.max_context_len, case.scale, ws)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).clone())
    assert torch.equal(outs[0], outs[1])
    pa.set_debug_checks(True)
    p = wl.multi_query_decode()
    pdev = place(p)
    pa.store_kv(pdev.step_k, pdev.step_v, pdev.step_slots, pdev.k_cache, pdev.v_cache)
    out = torch.empty((p.total_q_rows, 16, 128), dtype=torch.bfloat16, device="cuda")
    pa.prefill(out, pdev.q, pdev.cu_q, pdev.context_lens, p.max_q_len, pdev.k_cache, pdev.v_cache,
               pdev.block_table, p.scale,
               pa.alloc_prefill_workspace(p.batch, p.total_q_rows, p.max_q_len, 16, 8,
                                          p.max_blocks_per_seq))
    wsm = pa.alloc_decode_multi_workspace(p.batch, 4, 16, 8)
    pa.decode_multi(out, pdev.q, pdev.k_cache, pdev.v_cache, pdev.block_table, pdev.context_lens, 4,
                    p.max_context_len, p.scale, wsm)
    torch.cuda.synchronize()


def test_slot_past_the_pool(checks_on):
    k, v = pa.alloc_cache(4, 8, "cuda", fill_bits=wl.POISON_BF16)
    rows = wl.normal_bf16(80, 2, 0, 3 * 8 * 128).view(3, 8, 128).cuda()
    slots = torch.tensor([5, 4 * 256, -1], dtype=torch.int32, device="cuda")
    expect_precondition(lambda: pa.store_kv(rows, rows, slots, k, v), ["slot"])
    torch.cuda.synchronize()
    assert bool((k.view(torch.int16) == wl.POISON_BF16).all())  # nothing was stored


def _decode_call(case, dev, ctx=None, table=None):
    out = torch.full((case.batch, case.num_q_heads, 128), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    ws = pa.alloc_decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads)
    ctx = dev.context_lens if ctx is None else ctx
    table = dev.block_table if table is None else table

    def call():
        pa.decode(out, dev.q, dev.k_cache, dev.v_cache, table, ctx, case.max_context_len,
                  case.scale, ws)
    return call, out


def test_context_length_out_of_range(checks_on):
    case = wl.tiny_decode()
    dev = place(case)
    for bad in (case.max_context_len + 1, -3):
        ctx = dev.context_lens.clone()
        ctx[1] = bad
        call, out = _decode_call(case, dev, ctx=ctx)
        expect_precondition(call, ["context length"])
        torch.cuda.synchronize()
        assert bool(torch.isnan(out).all())


def test_block_table_entry_outside_the_pool(checks_on):
    case = wl.tiny_decode()
    dev = place(case)
    for bad in (case.num_blocks, -1):
        table = dev.block_table.clone()
        table[3, 1] = bad  # sequence 3 (257 tokens) uses two blocks
        call, out = _decode_call(case, dev, table=table)
        expect_precondition(call, ["block-table"])
        torch.cuda.synchronize()
        assert bool(torch.isnan(out).all())
    # entries past the blocks a sequence uses are not read: no error
    table = dev.block_table.clone()
    table[0, 1] = -1  # sequence 0 holds one token
    call, _ = _decode_call(case, dev, table=table)
    call()
    torch.cuda.synchronize()


def test_query_rows_inconsistent(checks_on):
    p = wl.make_case("rows", "prefill", 81, [300, 40, 700], 16, 8, q_lens=[300, 20, 5])
    dev = place(p)
    out = torch.full((p.total_q_rows, 16, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = pa.alloc_prefill_workspace(p.batch, p.total_q_rows, p.max_q_len, 16, 8,
                                    p.max_blocks_per_seq)

    def prefill(cu, ctx):
        pa.prefill(out, dev.q, cu, ctx, p.max_q_len, dev.k_cache, dev.v_cache, dev.block_table,
                   p.scale, ws)

    ctx = dev.context_lens.clone()
    ctx[1] = 10  # 20 query rows over 10 tokens
    expect_precondition(lambda: prefill(dev.cu_q, ctx), ["query rows"])
    cu = dev.cu_q.clone()
    cu[3] = cu[3] - 1  # last offset != rows of q
    expect_precondition(lambda: prefill(cu, dev.context_lens), ["query rows"])
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all())
    # pa_decode_multi: fewer cached tokens than rows per sequence
    m = wl.make_case("mrows", "prefill", 82, [8, 100], 16, 8, q_lens=[4, 4])
    mdev = place(m)
    mctx = mdev.context_lens.clone()
    mctx[0] = 3
    mout = torch.full((8, 16, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    wsm = pa.alloc_decode_multi_workspace(2, 4, 16, 8)
    expect_precondition(lambda: pa.decode_multi(mout, mdev.q, mdev.k_cache, mdev.v_cache,
                                                mdev.block_table, mctx, 4, m.max_context_len,
                                                m.scale, wsm), ["query rows"])
    torch.cuda.synchronize()
    assert bool(torch.isnan(mout).all())
