"""The seeded input generators: determinism, slicing, distribution, and the
block-assignment rules (fixed 256-token blocks; a sequence takes a new block at
256k+1 tokens; physical blocks from a seeded shuffle)."""

import math

import numpy as np
import torch

import workloads as wl


def test_generator_is_deterministic_and_sliceable():
    a = wl.normal_bf16(7, wl.STREAM_K, 0, 5000)
    b = wl.normal_bf16(7, wl.STREAM_K, 0, 5000)
    assert torch.equal(a, b)
    assert torch.equal(wl.normal_bf16(7, wl.STREAM_K, 1234, 100), a[1234:1334])
    assert not torch.equal(wl.normal_bf16(7, wl.STREAM_V, 0, 5000), a)
    assert not torch.equal(wl.normal_bf16(8, wl.STREAM_K, 0, 5000), a)


def test_generator_handles_indices_past_2_pow_32():
    x = wl.normal_bf16(3, wl.STREAM_K, (1 << 32) - 10, 20)
    y = wl.normal_bf16(3, wl.STREAM_K, 0, 20)
    assert not torch.equal(x, y)


def test_generator_is_standard_normal():
    x = wl.normal_bf16(1, wl.STREAM_Q, 0, 1 << 20).view(torch.bfloat16).double()
    assert torch.isfinite(x).all()
    assert abs(x.mean().item()) < 5e-3
    assert abs(x.std().item() - 1.0) < 5e-3
    # two-sided tail mass beyond 2 sigma ~ 4.55 %
    tail = (x.abs() > 2).double().mean().item()
    assert abs(tail - 0.0455) < 2e-3
    # odd-moment symmetry and neighbour independence
    assert abs(((x[1:] * x[:-1]).mean()).item()) < 5e-3


def test_q_multiplier_is_exact():
    c1 = wl.make_case("a", "decode", 9, [3, 4], 4, 2)
    c32 = wl.make_case("a", "decode", 9, [3, 4], 4, 2, q_mult=32.0)
    q1 = c1.q_all().view(torch.bfloat16).double()
    q32 = c32.q_all().view(torch.bfloat16).double()
    assert torch.equal(q1 * 32, q32)


def test_blocks_for_follows_256k_plus_1_rule():
    assert [wl.blocks_for(n) for n in (0, 1, 255, 256, 257, 512, 513, 131072)] == \
        [0, 1, 1, 1, 2, 2, 3, 512]


def test_pool_headroom_rule():
    assert wl.pool_size_with_headroom(64) == 71
    assert wl.pool_size_with_headroom(4096) == 4506
    assert wl.pool_size_with_headroom(10) == 11


def _check_tables(case):
    used = case.block_table[case.block_table >= 0]
    assert len(np.unique(used)) == len(used), "a physical block is shared"
    assert used.min() >= 0 and used.max() < case.num_blocks
    for b in range(case.batch):
        k = wl.blocks_for(int(case.context_lens[b]), case.block_size)
        assert np.all(case.block_table[b, :k] >= 0) and np.all(case.block_table[b, k:] == -1)
    slots = case.slot_mapping_all
    assert len(np.unique(slots)) == len(slots)
    assert slots.min() >= 0 and slots.max() < case.num_blocks * case.block_size


def test_configs_shapes_and_rules():
    t = wl.tiny_decode()
    assert list(t.context_lens) == [1, 255, 256, 257] and t.num_blocks == 8
    assert (t.num_q_heads, t.num_kv_heads, t.head_dim, t.block_size) == (16, 8, 128, 256)
    _check_tables(t)
    assert abs(t.scale - 1 / math.sqrt(128)) < 1e-15

    c2 = wl.qwen3_0_6b_decode()
    assert c2.batch == 64 and c2.context_lens.min() >= 512 and c2.context_lens.max() <= 4096
    assert c2.num_blocks == wl.pool_size_with_headroom(c2.used_blocks)
    _check_tables(c2)

    c3 = wl.qwen3_4b_decode()
    assert c3.batch == 256 and (c3.num_q_heads, c3.num_kv_heads) == (32, 8)
    assert c3.context_lens.min() >= 64 and c3.context_lens.max() <= 32768
    assert 1024 <= np.median(c3.context_lens) <= 4096
    _check_tables(c3)

    c4 = wl.prefill_8x2048()
    assert c4.total_q_rows == 16384 and c4.num_blocks == 71
    assert np.array_equal(c4.q_lens, c4.context_lens)
    _check_tables(c4)

    c5 = wl.long_context_decode()
    assert c5.total_kv_rows == 8 * 131072 and c5.num_blocks == 4506
    assert c5.max_blocks_per_seq == 512
    _check_tables(c5)

    c6 = wl.chunked_prefill_mixed()
    assert c6.batch == 72 and c6.total_q_rows == 64 + 8 * 512
    assert np.all(c6.q_lens[:64] == 1) and np.all(c6.q_lens[64:] == 512)
    assert np.all(c6.context_lens[64:] >= 512 + 512) and np.all(c6.context_lens[64:] <= 8192 + 512)
    _check_tables(c6)

    c7 = wl.multi_query_decode()
    assert c7.batch == 64 and np.all(c7.q_lens == 4) and c7.total_q_rows == 256
    _check_tables(c7)

    c8 = wl.long_prefix_chunk()
    assert c8.batch == 1 and c8.total_q_rows == 512 and int(c8.context_lens[0]) == 65536 + 512
    assert c8.max_blocks_per_seq == (65536 + 512) // 256
    _check_tables(c8)


def test_step_and_history_rows_partition_the_cache():
    c = wl.make_case("x", "decode", 5, [1, 4, 300], 4, 2)
    rows = np.sort(np.concatenate([c.step_rows(), c.history_rows()]))
    assert np.array_equal(rows, np.arange(c.total_kv_rows))
    assert list(c.step_rows()) == [0, 4, 304]
    p = wl.make_case("y", "prefill", 5, [5, 7], 2, 1, q_lens=[2, 7])
    assert list(p.step_rows()) == [3, 4, 5, 6, 7, 8, 9, 10, 11]
