"""Placing a seeded case in device memory through the library: NaN-poisoned
caches, the case's K/V generated on the device, the history stored with
pa_store_kv.  Used by the GPU tests and the benchmark; it imports only the
library, the seeded input generators and torch."""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

import paged_kv_cache_237_amd as pa
import workloads as wl


@dataclasses.dataclass
class DeviceCase:
    case: wl.PagedCase
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    context_lens: torch.Tensor
    q: torch.Tensor
    step_k: torch.Tensor
    step_v: torch.Tensor
    step_slots: torch.Tensor
    cu_q: torch.Tensor


def place(case: wl.PagedCase, device="cuda", store_history=True) -> DeviceCase:
    """Allocate NaN-poisoned caches, generate the case's K/V on the device and
    store the history (everything but the step's new tokens) with
    pa_store_kv."""
    k_cache, v_cache = pa.alloc_cache(case.num_blocks, case.num_kv_heads, device,
                                      fill_bits=wl.POISON_BF16)
    slots_all = torch.from_numpy(case.slot_mapping_all.copy()).to(device)
    step_rows = torch.from_numpy(case.step_rows()).to(device)
    if case.total_kv_rows:
        k_all = case.k_rows(0, case.total_kv_rows, device)
        v_all = case.v_rows(0, case.total_kv_rows, device)
        if store_history:
            hist_slots = slots_all.clone()
            hist_slots[step_rows] = -1
            pa.store_kv(k_all, v_all, hist_slots, k_cache, v_cache)
        step_k = k_all[step_rows].contiguous()
        step_v = v_all[step_rows].contiguous()
        del k_all, v_all
    else:
        step_k = torch.empty((0, case.num_kv_heads, case.head_dim), dtype=torch.int16, device=device)
        step_v = step_k.clone()
    return DeviceCase(
        case=case, k_cache=k_cache, v_cache=v_cache,
        block_table=torch.from_numpy(case.block_table.copy()).to(device),
        context_lens=torch.from_numpy(case.context_lens.copy()).to(device),
        q=case.q_all(device), step_k=step_k, step_v=step_v,
        step_slots=slots_all[step_rows].contiguous(),
        cu_q=torch.from_numpy(case.q_offsets.astype(np.int32)).to(device))


def new_rows(dev: DeviceCase):
    """k_new / v_new [B, Hkv, 128] for pa_decode_append: the step token of each
    non-empty sequence (one per sequence, in batch order), zeros for empty
    sequences."""
    case = dev.case
    k = torch.zeros((case.batch, case.num_kv_heads, case.head_dim), dtype=dev.step_k.dtype,
                    device=dev.step_k.device)
    v = torch.zeros_like(k)
    nz = torch.from_numpy(np.nonzero(case.context_lens > 0)[0]).to(k.device)
    k[nz] = dev.step_k
    v[nz] = dev.step_v
    return k, v
