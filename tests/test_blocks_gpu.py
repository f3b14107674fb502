"""Whole-block copies on the GPU: pa_copy_blocks (copy-on-write inside a pool)
against the float64 oracle's block copy, byte for byte over whole poisoned
pools; at full size against the definition (block dst afterwards holds the
bytes block src held before, every other block is unchanged); and
pa_swap_blocks between the device pool and a pinned host pool and back."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_237_amd as pa
import workloads as wl
from paged_harness import oracle_pools, place

pytestmark = pytest.mark.gpu


def pick_pairs(case, rng, n_pairs, n_invalid=3):
    """n_pairs (src, dst): sources among the used blocks, destinations among
    the free ones (distinct, never a source), plus skipped pairs (-1 padding,
    src == dst, an index past the pool) spread through the list."""
    used = np.unique(case.block_table[case.block_table >= 0])
    free = np.setdiff1d(np.arange(case.num_blocks), used)
    n_pairs = min(n_pairs, len(free))
    src = rng.choice(used, size=n_pairs, replace=True)
    dst = rng.choice(free, size=n_pairs, replace=False)
    pairs = np.stack([src, dst], axis=1).astype(np.int32)
    junk = np.array([[-1, int(free[0])], [int(used[0]), int(used[0])],
                     [int(used[0]), case.num_blocks]], dtype=np.int32)[:n_invalid]
    pairs = np.concatenate([pairs, junk])
    return pairs[rng.permutation(len(pairs))]


def pool_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_copy_blocks_matches_oracle_over_whole_pools():
    case = wl.make_case("copy", "decode", 61, [1, 255, 256, 257, 700, 1024], 16, 8,
                        num_blocks=24)
    print(f"[copy_blocks] {case.name} blocks={case.num_blocks}", flush=True)
    dev = place(case)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    pairs = pick_pairs(case, np.random.default_rng(61), 8)
    in_pool = pairs[(pairs < case.num_blocks).all(axis=1)]
    assert pa.validate_block_pairs(in_pool, case.num_blocks) == 0
    assert pa.validate_block_pairs(pairs, case.num_blocks) == -7  # the past-the-pool pair
    pa.copy_blocks(dev.k_cache, dev.v_cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    kp, vp = oracle_pools(case)
    oracle.copy_blocks(kp, vp, pairs)
    assert np.array_equal(pool_bits(dev.k_cache), kp)
    assert np.array_equal(pool_bits(dev.v_cache), vp)


def test_copy_blocks_full_size_definition():
    case = wl.qwen3_0_6b_decode()
    print(f"[copy_blocks] {case.name} blocks={case.num_blocks}", flush=True)
    dev = place(case)
    pairs = pick_pairs(case, np.random.default_rng(62), 64)
    in_pool = pairs[(pairs < case.num_blocks).all(axis=1)]
    assert pa.validate_block_pairs(in_pool, case.num_blocks) == 0
    k0, v0 = dev.k_cache.clone(), dev.v_cache.clone()
    pa.copy_blocks(dev.k_cache, dev.v_cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    ek, ev = k0.clone(), v0.clone()
    for s, d in pairs:
        if 0 <= s < case.num_blocks and 0 <= d < case.num_blocks and s != d:
            ek[d] = k0[s]
            ev[d] = v0[s]
    assert torch.equal(dev.k_cache.view(torch.int16), ek.view(torch.int16))
    assert torch.equal(dev.v_cache.view(torch.int16), ev.view(torch.int16))


def test_empty_pair_list_is_a_no_op():
    k, v = pa.alloc_cache(4, 2, "cuda", fill_bits=wl.POISON_BF16)
    pa.copy_blocks(k, v, torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.all(pool_bits(k) == wl.POISON_BF16)


def test_swap_out_and_back_in():
    case = wl.make_case("swap", "decode", 63, [300, 1000, 2049, 64], 16, 8)
    print(f"[swap_blocks] {case.name} blocks={case.num_blocks}", flush=True)
    dev = place(case)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    used = np.unique(case.block_table[case.block_table >= 0]).astype(np.int32)
    host_blocks = len(used) + 2
    hk = torch.empty((host_blocks,) + tuple(dev.k_cache.shape[1:]), dtype=torch.bfloat16,
                     pin_memory=True)
    hv = torch.empty((host_blocks,) + tuple(dev.v_cache.shape[1:]), dtype=torch.bfloat16,
                     pin_memory=True)
    hk.view(torch.int16).fill_(0)
    hv.view(torch.int16).fill_(0)
    # swap out: used block used[i] -> host block i + 1 (a run and some jumps)
    out_pairs = np.stack([used, np.arange(1, len(used) + 1, dtype=np.int32)], axis=1)
    pa.swap_blocks(dev.k_cache, dev.v_cache, hk, hv, out_pairs)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(case)
    hkb, hvb = pool_bits(hk), pool_bits(hv)
    for s, d in out_pairs:
        assert np.array_equal(hkb[d], kp[s]) and np.array_equal(hvb[d], vp[s])
    assert np.all(hkb[0] == 0) and np.all(hkb[-1] == 0)
    # swap back in, reversed order, into a fresh device pool
    k2, v2 = pa.alloc_cache(case.num_blocks, case.num_kv_heads, "cuda",
                            fill_bits=wl.POISON_BF16)
    in_pairs = out_pairs[::-1, ::-1].copy()
    pa.swap_blocks(hk, hv, k2, v2, in_pairs)
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits(k2), kp) and np.array_equal(pool_bits(v2), vp)
