"""pa_store_kv on the GPU against the oracle's store: the cache bytes must be
identical (a bit copy), untouched slots keep their NaN poison, negative slots
are skipped."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_237_amd as pa
import workloads as wl
from paged_harness import compare_pools_bytes, oracle_pools, place

pytestmark = pytest.mark.gpu


def _store_all(case):
    """Place nothing, then store every token of the case in one call."""
    dev = place(case, store_history=False)
    slots = torch.from_numpy(case.slot_mapping_all.copy()).cuda()
    k_all = case.k_rows(0, case.total_kv_rows, "cuda")
    v_all = case.v_rows(0, case.total_kv_rows, "cuda")
    pa.store_kv(k_all, v_all, slots, dev.k_cache, dev.v_cache)
    torch.cuda.synchronize()
    return dev


def test_store_tiny_decode_step_bit_exact():
    case = wl.tiny_decode()
    print(f"[store] {case.name}", flush=True)
    dev = place(case)
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    torch.cuda.synchronize()
    kp, vp = oracle_pools(case)
    compare_pools_bytes(dev, kp, vp)


@pytest.mark.parametrize("lens", [[1], [64, 65, 300], [255, 256, 257, 511, 512, 513], [1000, 7, 0, 33]])
@pytest.mark.parametrize("hkv", [1, 2, 8])
def test_store_ragged_bit_exact(lens, hkv):
    case = wl.make_case("ragged", "prefill", 11, lens, hkv, hkv, num_blocks=None)
    print(f"[store] lens={lens} hkv={hkv}", flush=True)
    dev = _store_all(case)
    kp, vp = oracle_pools(case)
    compare_pools_bytes(dev, kp, vp)


def test_store_skips_negative_and_out_of_pool_slots():
    case = wl.make_case("neg", "prefill", 12, [300, 200], 8, 8)
    print("[store] negative slots", flush=True)
    dev = place(case, store_history=False)
    slots_np = case.slot_mapping_all.copy()
    rng = np.random.default_rng(12)
    drop = rng.choice(len(slots_np), size=60, replace=False)
    slots_np[drop[:30]] = -1
    slots_np[drop[30:]] = -123456
    k_all = case.k_rows(0, case.total_kv_rows, "cuda")
    v_all = case.v_rows(0, case.total_kv_rows, "cuda")
    pa.store_kv(k_all, v_all, torch.from_numpy(slots_np).cuda(), dev.k_cache, dev.v_cache)
    torch.cuda.synchronize()
    kp, vp = oracle.new_pools(case.num_blocks, 8, 128, 256, wl.POISON_BF16)
    oracle.store_kv(kp, vp, wl.bits_to_numpy(k_all), wl.bits_to_numpy(v_all), slots_np)
    compare_pools_bytes(dev, kp, vp)


def test_store_prefill_8x2048_bit_exact():
    case = wl.prefill_8x2048()
    print(f"[store] {case.name}", flush=True)
    dev = _store_all(case)
    kp, vp = oracle_pools(case)
    compare_pools_bytes(dev, kp, vp)


def test_store_empty_is_a_no_op():
    k, v = pa.alloc_cache(2, 8, "cuda", fill_bits=wl.POISON_BF16)
    e = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    pa.store_kv(e, e, torch.empty(0, dtype=torch.int32, device="cuda"), k, v)
    torch.cuda.synchronize()
    assert bool((k.view(torch.int16) == wl.POISON_BF16).all())
