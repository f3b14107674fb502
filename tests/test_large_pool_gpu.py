"""Pools larger than 4 GiB per cache, with every used block past the 4 GiB
line: the store, decode, decode_append, decode_multi, prefill (direct and
context-split) and block-copy kernels all address the caches with 64-bit
offsets, which a pool of this size checks (a 32-bit byte or element offset
would wrap and read or write the wrong block).  Attention outputs are held to
the usual bar against the float64 oracle; cache contents are compared byte
for byte on the rows the oracle defines, with the NaN poison still in every
row past a context."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_237_amd as pa
import workloads as wl
from device_case import new_rows
from paged_harness import bf16_out_to_f64, compare, oracle_pools, place

pytestmark = pytest.mark.gpu

HKV = 8
BLOCK_BYTES = HKV * wl.BLOCK_SIZE * wl.HEAD_DIM * 2  # one block of one cache
FIRST_HIGH = (1 << 32) // BLOCK_BYTES                 # first block starting at 4 GiB
NUM_BLOCKS = FIRST_HIGH + 808                         # 4.7 GB per cache


def high_case(name, kind, seed, ctx, hq, q_lens=None):
    """A seeded case whose blocks are drawn (shuffled) from the last blocks of
    the pool: from 8 blocks below the 4 GiB line to the end."""
    case = wl.make_case(name, kind, seed, ctx, hq, HKV, q_lens=q_lens, num_blocks=NUM_BLOCKS)
    rng = np.random.default_rng(seed + 1000)
    perm = rng.permutation(np.arange(FIRST_HIGH - 8, NUM_BLOCKS, dtype=np.int32))
    table = np.full_like(case.block_table, -1)
    pos = 0
    for b, n in enumerate(case.context_lens):
        k = wl.blocks_for(int(n))
        table[b, :k] = perm[pos:pos + k]
        pos += k
    assert pos <= perm.shape[0]
    return dataclasses.replace(case, block_table=table)


def check_cache_rows(dev, case, kp, vp):
    """Every cached row of every sequence holds the oracle's bytes; rows past
    a context still hold the poison."""
    for b in range(case.batch):
        n = int(case.context_lens[b])
        for i in range(wl.blocks_for(n)):
            blk = int(case.block_table[b, i])
            rows = min(wl.BLOCK_SIZE, n - i * wl.BLOCK_SIZE)
            kd = wl.bits_to_numpy(dev.k_cache[blk].view(torch.int16))
            vd = wl.bits_to_numpy(dev.v_cache[blk].view(torch.int16))
            assert np.array_equal(kd[:, :, :rows], kp[blk][:, :, :rows]), (b, i, blk)
            assert np.array_equal(vd[:, :rows], vp[blk][:, :rows]), (b, i, blk)
            assert np.all(kd[:, :, rows:] == wl.POISON_BF16), (b, i, blk)
            assert np.all(vd[:, rows:] == wl.POISON_BF16), (b, i, blk)


CTX = [1, 300, 1000, 2048, 257, 4097]


@pytest.mark.parametrize("hq", [16, 32])
def test_decode_and_store_past_4gib(hq):
    case = high_case(f"high_decode_{hq}", "decode", 71, CTX, hq)
    print(f"[large_pool] decode Hq={hq} blocks {int(case.block_table.max())} of {NUM_BLOCKS}",
          flush=True)
    used = case.block_table[case.block_table >= 0]
    assert (used >= FIRST_HIGH).mean() > 0.9 and int(used.max()) < NUM_BLOCKS
    dev = place(case)
    out = torch.empty((case.batch, hq, wl.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    ws = pa.alloc_decode_workspace(case.batch, hq, HKV)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    pa.decode(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens,
              case.max_context_len, case.scale, ws)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(case, poison=False)
    check_cache_rows(dev, case, kp, vp)
    ref = oracle.decode(wl.bits_to_numpy(case.q_all()), kp, vp, case.block_table,
                        case.context_lens, case.scale)
    compare(bf16_out_to_f64(out), ref, case.name)


def test_decode_append_past_4gib():
    case = high_case("high_append", "decode", 72, CTX, 16)
    print("[large_pool] decode_append", flush=True)
    dev = place(case)
    k_new, v_new = new_rows(dev)
    out = torch.empty((case.batch, 16, wl.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    ws = pa.alloc_decode_workspace(case.batch, 16, HKV)
    pa.decode_append(out, dev.q, k_new, v_new, dev.k_cache, dev.v_cache, dev.block_table,
                     dev.context_lens, case.max_context_len, case.scale, ws)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(case, poison=False)
    check_cache_rows(dev, case, kp, vp)
    ref = oracle.decode(wl.bits_to_numpy(case.q_all()), kp, vp, case.block_table,
                        case.context_lens, case.scale)
    compare(bf16_out_to_f64(out), ref, case.name)


def test_decode_multi_past_4gib():
    ql = 3
    case = high_case("high_multi", "prefill", 73, [3, 300, 1000, 2048, 257, 4097], 16,
                     q_lens=[ql] * 6)
    print("[large_pool] decode_multi", flush=True)
    dev = place(case)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    out = torch.full((case.batch * ql, 16, wl.HEAD_DIM), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    ws = pa.alloc_decode_multi_workspace(case.batch, ql, 16, HKV)
    pa.decode_multi(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens, ql,
                    case.max_context_len, case.scale, ws)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(case, poison=False)
    q = wl.bits_to_numpy(case.q_all())
    ref = np.concatenate([
        oracle.prefill_seq(q[b * ql:(b + 1) * ql], kp, vp, case.block_table[b],
                           int(case.context_lens[b]), case.scale) for b in range(case.batch)])
    compare(bf16_out_to_f64(out), ref, case.name)


@pytest.mark.parametrize("ctx,q_lens", [
    (CTX, [1, 300, 200, 512, 257, 256]),  # one launch, no context split
    ([8192], [128]),                      # few query blocks: context split + merge kernel
])
def test_prefill_past_4gib(ctx, q_lens):
    case = high_case(f"high_prefill_{len(ctx)}", "prefill", 74, ctx, 16, q_lens=q_lens)
    print(f"[large_pool] prefill ctx={ctx} q_lens={q_lens}", flush=True)
    dev = place(case)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    out = torch.full((case.total_q_rows, 16, wl.HEAD_DIM), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    ws = pa.alloc_prefill_workspace(case.batch, case.total_q_rows, case.max_q_len, 16, HKV,
                                    case.max_blocks_per_seq)
    pa.prefill(out, dev.q, dev.cu_q, dev.context_lens, case.max_q_len, dev.k_cache, dev.v_cache,
               dev.block_table, case.scale, ws)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(case, poison=False)
    check_cache_rows(dev, case, kp, vp)
    ref = oracle.prefill(wl.bits_to_numpy(case.q_all()), case.q_offsets, case.context_lens, kp, vp,
                         case.block_table, case.scale)
    compare(bf16_out_to_f64(out), ref, case.name)


def test_copy_blocks_past_4gib():
    """Copy-on-write pairs among high blocks: each destination block becomes a
    byte copy of its source (poisoned tail rows included); sources and every
    other used block are unchanged."""
    case = high_case("high_copy", "decode", 75, CTX, 16)
    print("[large_pool] copy_blocks", flush=True)
    dev = place(case)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    used = case.block_table[case.block_table >= 0]
    free = np.setdiff1d(np.arange(FIRST_HIGH, NUM_BLOCKS, dtype=np.int32), used)
    rng = np.random.default_rng(76)
    src = rng.choice(used, size=12, replace=False).astype(np.int32)
    dst = rng.choice(free, size=12, replace=False).astype(np.int32)
    assert int(dst.max()) >= FIRST_HIGH
    before_k = dev.k_cache[torch.from_numpy(used.astype(np.int64)).cuda()].clone()
    before_v = dev.v_cache[torch.from_numpy(used.astype(np.int64)).cuda()].clone()
    pairs = torch.from_numpy(np.stack([src, dst], axis=1)).cuda()
    pa.copy_blocks(dev.k_cache, dev.v_cache, pairs)
    torch.cuda.synchronize()
    for s, d in zip(src.tolist(), dst.tolist()):
        assert torch.equal(dev.k_cache[d].view(torch.int16), dev.k_cache[s].view(torch.int16)), (s, d)
        assert torch.equal(dev.v_cache[d].view(torch.int16), dev.v_cache[s].view(torch.int16)), (s, d)
    ui = torch.from_numpy(used.astype(np.int64)).cuda()
    assert torch.equal(dev.k_cache[ui].view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(dev.v_cache[ui].view(torch.int16), before_v.view(torch.int16))
